// Device helpers for the verification kernels (gfx950, wave64).
//
// Loads: logits arrive as bf16 bit patterns or fp32; a "group" is 8 consecutive
// elements (one 16-byte load for bf16, two for fp32). bf16 widens to fp32
// exactly by a 16-bit shift.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <float.h>
#include <math.h>

namespace sv {

constexpr int kThreads = 256;  // 4 wave64 per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kGroup = 8;      // elements per group

// ---------------------------------------------------------------- loads
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// One aligned group of 8 logits starting at element offset `e` of `p`.
__device__ __forceinline__ void load_group(const uint16_t* __restrict__ p, size_t e, float x[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p + e);
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}
__device__ __forceinline__ void load_group(const float* __restrict__ p, size_t e, float x[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p + e);
  const float4 b = *reinterpret_cast<const float4*>(p + e + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ float load_one(const uint16_t* __restrict__ p, size_t e) {
  return __uint_as_float(static_cast<uint32_t>(p[e]) << 16);
}
__device__ __forceinline__ float load_one(const float* __restrict__ p, size_t e) { return p[e]; }

// ---------------------------------------------------------------- math
__device__ __forceinline__ float fast_exp2(float y) { return __builtin_amdgcn_exp2f(y); }

// Merge two (max, sum exp2((x - max) * k)) partial states.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2, float k2) {
  const float M = fmaxf(m, m2);
  s = s * fast_exp2((m - M) * k2) + s2 * fast_exp2((m2 - M) * k2);
  m = M;
}

// ---------------------------------------------------------------- wave / block reductions
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int wave_min_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

// Block-wide sum of N doubles; result valid in every thread. `lds` holds kWaves*N.
template <int N>
__device__ __forceinline__ void block_sum(double (&v)[N], double* lds) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = wave_sum(v[i]);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) lds[w * N + i] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    double t = 0.0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) t += lds[k * N + i];
    v[i] = t;
  }
  __syncthreads();
}

__device__ __forceinline__ float block_max(float v, float* lds) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if (lane == 0) lds[w] = v;
  __syncthreads();
  float t = lds[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) t = fmaxf(t, lds[k]);
  __syncthreads();
  return t;
}

__device__ __forceinline__ int block_min_int(int v, int* lds) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_min_int(v);
  if (lane == 0) lds[w] = v;
  __syncthreads();
  int t = lds[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) t = min(t, lds[k]);
  __syncthreads();
  return t;
}
__device__ __forceinline__ int block_max_int(int v, int* lds) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_max_int(v);
  if (lane == 0) lds[w] = v;
  __syncthreads();
  int t = lds[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) t = max(t, lds[k]);
  __syncthreads();
  return t;
}

// Exclusive block scan of one double per thread (thread order); returns the
// prefix of the threads before this one. `lds` holds kWaves doubles.
__device__ __forceinline__ double block_excl_scan(double v, double* lds) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double n = __shfl_up(inc, o);
    if (lane >= o) inc += n;
  }
  if (lane == 63) lds[w] = inc;
  __syncthreads();
  double base = 0.0;
  for (int k = 0; k < w; ++k) base += lds[k];
  __syncthreads();
  return base + inc - v;
}

// Greedy partial: (value, index) with the larger value winning, lowest index on ties.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

// Largest b in [0, B) with cu[b] <= d, for a non-decreasing cu with cu[0] = 0
// (B <= 65536). Every thread of the block calls it; result valid in all threads.
__device__ __forceinline__ int seq_of_row(const int32_t* __restrict__ cu, int B, int d) {
  const int step = (B + kThreads - 1) / kThreads;
  const int t = threadIdx.x;
  const int p1 = t * step;
  const int c1 = __syncthreads_count(p1 < B && cu[p1] <= d);
  const int lo = max(0, (c1 - 1) * step);
  const int p2 = lo + t;
  const int c2 = __syncthreads_count(t < step && p2 < B && cu[p2] <= d);
  return min(B - 1, max(0, lo + c2 - 1));
}

}  // namespace sv

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
__device__ __forceinline__ float bf16_word_half(uint32_t w, int hi) { return hi ? bf16_hi(w) : bf16_lo(w); }

// 16-byte load; NT marks it nontemporal (streamed data that is not read again soon).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ uint4 load16(const uint4* p) {
  if constexpr (NT) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *p;
  }
}

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

// 2^(Z/N) in float64 for Z in units of 1/N octave, N = 2^SV_EXP_LOG2N table entries.
// With n = rint(Z) = N k + j (0 <= j < N) and f = Z - n (exact, |f| <= 1/2):
// 2^(Z/N) = 2^k * 2^(j/N) * e^(f c), c = ln2/N, e^(f c) from a short Taylor
// polynomial: degree 3 for N = 256 (relative error below 1.5e-13), degree 2 for
// N = 2048 (below 1e-12). rint comes from adding 1.5 * 2^52, whose sum keeps n in
// its low 32 bits. `tab` holds 2^(j/N). Arguments below -3e8 (and -inf) give 0;
// results below 2^-1022 come out subnormal.
#ifndef SV_EXP_LOG2N
#define SV_EXP_LOG2N 8
#endif
constexpr int kExpN = 1 << SV_EXP_LOG2N;
constexpr double kExpScale = static_cast<double>(kExpN);  // Z = kExpScale * octaves

__device__ __forceinline__ double exp2_tab(double Z, const double* tab) {
  Z = fmax(Z, -3.0e8);
  const double t = Z + 6755399441055744.0;
  const double n = t - 6755399441055744.0;
  const double f = Z - n;
#if SV_EXP_LOG2N == 8
  double p = fma(f, 3.3083026805413713e-09, 3.6655655969101062e-06);  // c^3/6, c^2/2
  p = fma(f, p, 2.7076061740622863e-03);                              // c
  p = fma(f, p, 1.0);
#elif SV_EXP_LOG2N == 11
  double p = fma(f, 5.7274462451720440e-08, 3.3845077175778579e-04);  // c^2/2, c
  p = fma(f, p, 1.0);
#else
#error "SV_EXP_LOG2N must be 8 or 11"
#endif
  const int ni = __double2loint(t);
  return ldexp(tab[ni & (kExpN - 1)] * p, ni >> SV_EXP_LOG2N);
}

// Fill tab[0..N-1] with 2^(j/N) (all threads of the block); caller syncs.
__device__ __forceinline__ void exp_table_init(double* tab) {
  for (int j = threadIdx.x; j < kExpN; j += blockDim.x) tab[j] = exp2(static_cast<double>(j) / kExpScale);
}

// Wave-wide max of a float through DPP row permutations and four lane reads (no LDS
// traffic); the result is wave-uniform.
__device__ __forceinline__ float wave_max_dpp(float v) {
  int x = __float_as_int(v);
  // within rows of 16 lanes: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false))));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(x, 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(x, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(x, 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(x, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// ---------------------------------------------------------------- DPP forms (no LDS round trip)
// DPP controls used below: quad_perm [1,0,3,2] 0xB1, quad_perm [2,3,0,1] 0x4E,
// row_half_mirror 0x141, row_mirror 0x140, row_shr:n 0x110 + n, row_bcast:15 0x142,
// row_bcast:31 0x143. Lanes of disabled rows (and, with BOUND, lanes whose source lies
// outside the row) receive `old`.
template <int CTRL, int ROWS = 0xF, bool BOUND = false>
__device__ __forceinline__ double dpp_d(double v, double old) {
  const int lo = __builtin_amdgcn_update_dpp(__double2loint(old), __double2loint(v), CTRL, ROWS, 0xF, BOUND);
  const int hi = __builtin_amdgcn_update_dpp(__double2hiint(old), __double2hiint(v), CTRL, ROWS, 0xF, BOUND);
  return __hiloint2double(hi, lo);
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ double readlane_d(double v, int l) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                          __builtin_amdgcn_readlane(__double2loint(v), l));
}
// Sum over the wave; the result is wave-uniform.
__device__ __forceinline__ double wave_sum_dpp(double v) {
  v += dpp_d<0xB1>(v, 0.0);
  v += dpp_d<0x4E>(v, 0.0);
  v += dpp_d<0x141>(v, 0.0);
  v += dpp_d<0x140>(v, 0.0);
  return (readlane_d(v, 0) + readlane_d(v, 16)) + (readlane_d(v, 32) + readlane_d(v, 48));
}
// Inclusive prefix sum over the lanes of the wave, in lane order.
__device__ __forceinline__ double wave_incl_scan_dpp(double v) {
  v += dpp_d<0x111, 0xF, true>(v, 0.0);
  v += dpp_d<0x112, 0xF, true>(v, 0.0);
  v += dpp_d<0x114, 0xF, true>(v, 0.0);
  v += dpp_d<0x118, 0xF, true>(v, 0.0);
  v += dpp_d<0x142, 0xA>(v, 0.0);  // row 0's total into row 1, row 2's into row 3
  v += dpp_d<0x143, 0xC>(v, 0.0);  // lane 31's total into rows 2 and 3
  return v;
}
__device__ __forceinline__ int wave_min_int_dpp(int x) {
  x = min(x, dpp_i<0xB1>(x));
  x = min(x, dpp_i<0x4E>(x));
  x = min(x, dpp_i<0x141>(x));
  x = min(x, dpp_i<0x140>(x));
  return min(min(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             min(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}
__device__ __forceinline__ int wave_max_int_dpp(int x) {
  x = max(x, dpp_i<0xB1>(x));
  x = max(x, dpp_i<0x4E>(x));
  x = max(x, dpp_i<0x141>(x));
  x = max(x, dpp_i<0x140>(x));
  return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
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

// Block-wide reductions over NW waves (blockDim.x == 64 * NW); the result is
// valid in every thread. Each call ends with a barrier, so `lds` may be reused.
template <int NW, int N>
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
    for (int k = 0; k < NW; ++k) t += lds[k * N + i];
    v[i] = t;
  }
  __syncthreads();
}

template <int NW>
__device__ __forceinline__ float block_max(float v, float* lds) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if (lane == 0) lds[w] = v;
  __syncthreads();
  float t = lds[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) t = fmaxf(t, lds[k]);
  __syncthreads();
  return t;
}

template <int NW>
__device__ __forceinline__ double block_max_d(double v, double* lds) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  if (lane == 0) lds[w] = v;
  __syncthreads();
  double t = lds[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) t = fmax(t, lds[k]);
  __syncthreads();
  return t;
}

template <int NW>
__device__ __forceinline__ int block_min_int(int v, int* lds) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_min_int(v);
  if (lane == 0) lds[w] = v;
  __syncthreads();
  int t = lds[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) t = min(t, lds[k]);
  __syncthreads();
  return t;
}

template <int NW>
__device__ __forceinline__ int block_max_int(int v, int* lds) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_max_int(v);
  if (lane == 0) lds[w] = v;
  __syncthreads();
  int t = lds[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) t = max(t, lds[k]);
  __syncthreads();
  return t;
}

// Exclusive scan of one double per lane within a wave (lane order).
__device__ __forceinline__ double wave_excl_scan(double v) {
  const int lane = threadIdx.x & 63;
  double inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double n = __shfl_up(inc, o);
    if (lane >= o) inc += n;
  }
  const double prev = __shfl_up(inc, 1);
  return lane == 0 ? 0.0 : prev;
}

// Exclusive block scan of one double per thread (thread order); returns the
// sum of the values of the threads before this one. `lds` holds NW doubles.
template <int NW>
__device__ __forceinline__ double block_excl_scan(double v, double* lds) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const double ex = wave_excl_scan(v);
  if (lane == 63) lds[w] = ex + v;
  __syncthreads();
  double base = 0.0;
  for (int k = 0; k < w; ++k) base += lds[k];
  __syncthreads();
  return base + ex;
}

// Greedy partial: (value, index) with the larger value winning, lowest index on ties.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

// NaN watch of the greedy rows: a NaN-propagating running max (IEEE maximum, one
// v_maximum3_f32 per two entries) of every entry a lane reads, NaN afterwards iff one
// of the entries was NaN. Start it at -inf.
__device__ __forceinline__ float nan_watch(float t, const float (&x)[8]) {
#pragma unroll
  for (int j = 0; j < 8; j += 2)
    t = __builtin_elementwise_maximum(t, __builtin_elementwise_maximum(x[j], x[j + 1]));
  return t;
}
__device__ __forceinline__ float nan_watch1(float t, float x) { return __builtin_elementwise_maximum(t, x); }
// Raises `bit` in *err (once per wave) when a lane's watch holds NaN. Every lane of the
// wave calls it.
__device__ __forceinline__ void flag_nan(float t, int* err, int bit) {
  if (__ballot(t != t) != 0 && (threadIdx.x & 63) == 0) atomicOr(err, bit);
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

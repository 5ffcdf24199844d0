// libspecverify: batched verification step of speculative sampling, HIP for gfx950.
//
// Sources (what is computed):
//   [P1] "Speculative Decoding" (atonlee.tistory.com/330), ch.2 (round structure:
//        k accepted + 1 replacement or bonus token, later drafts discarded) and
//        ch.3 (accept iff r < min(1, p/q); residual norm(max(0, p - q)); greedy at T = 0).
//   [P2] "Speculative Decoding으로 LLM 추론 속도 높이기" (donmain.dev), "품질은 rejection
//        sampling이 지킨다" (p >= q accepts outright, residual draw).
//   [P3] "Fast Inference from Transformers via Speculative Decoding" (notes), 방법론 상세,
//        단계 3 (alpha_i, first-rejection residual, bonus from p(. | x_{1:n+gamma})).
//   [P4] "투기적 디코딩 — 초안 모델을 무엇으로 세울 것인가" (ailab.paldyn.com), "출력이
//        변하지 않는다는 것이 핵심이다" (greedy reduces to argmax equality).
//
// Pipeline per call (three launches on the caller's stream, no host sync):
//   1. k_rowstats / k_rowargmax: one read of every judged (draft) target row,
//      split over `split` workgroups per row. Sampling: online max and
//      sum exp((l - m)/T) in fp32 (p = softmax(l / T)). Greedy: max and its
//      lowest index. Partials go to the workspace.
//   2. k_sample_chunks / k_greedy_chunks, grid = B x nc (4096-element chunks of
//      the vocabulary). Prologue: merge the partials of the sequence's rows, run
//      the accept test of every draft position (p(x) in fp64), find the first
//      rejection n_b. Body: one fp64 sweep of this chunk of the single row that
//      will be drawn from: the rejected row (residual) or row gamma_b (bonus).
//      The residual sweep defers normalisation: with e(v) = exp((l(v) - m)/T),
//      v is positive iff e(v) > q(v) * Z32 (Z32 from step 1) and the chunk
//      keeps E = sum_pos e, Q = sum_pos q, Zc = sum e. The bonus sweep keeps a
//      chunk max and sum exp((l - m_c)/T). Greedy keeps the chunk argmax of row
//      gamma_b only when every draft was accepted.
//   3. k_sample_finalize / k_greedy_finalize, grid = B: combine chunk sums
//      (Z64 = sum Zc, R_c = E_c / Z64 - Q_c, S = sum R_c), locate the chunk where
//      the prefix crosses t = u * S, re-sweep that chunk with an fp64 block scan
//      and emit the first token whose inclusive prefix exceeds t.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdio.h>
#include <stdint.h>
#include <string.h>

#include <climits>
#include <new>

#include "spec_verify.h"
#include "sv_device.h"

using namespace sv;

namespace {

constexpr int kChunkGroups = 2;                            // groups per thread per chunk
constexpr int kChunk = kThreads * kGroup * kChunkGroups;   // 4096 vocabulary entries
constexpr int kMaxSplit = 16;
constexpr int kMaxGamma = 1024;
constexpr int kMaxRaggedBatch = 65536;  // row -> sequence search limit
constexpr int kMaxBatch = 1 << 24;
constexpr int kUnroll = 4;  // groups in flight per thread in the row-stats loop

struct RowStat { float m; float z; };  // sampling: max raw logit, sum exp((l - m)/T); greedy: max, index bits
struct SeqInfo { int n; int mode; float m; float z; int tok; int g; int base; int pad; };
enum { MODE_RESIDUAL = 0, MODE_BONUS = 1, MODE_GREEDY = 2, MODE_INVALID = 3 };

struct Args {
  const void* logits;
  const float* q;
  const int32_t* ids;
  const float* u;
  const int32_t* cu;
  int32_t* acc;
  int32_t* emitted;
  float* rsum;
  float* pdraft;
  RowStat* p1;
  double* csum;   // [B][nc][3]
  SeqInfo* info;  // [B]
  int* err;
  int B, gamma, V, R, split, span, nc, max_gamma;
  float k2;       // log2(e) / T
  double invT;    // 1 / T
};

__device__ __forceinline__ bool finite_pos(float z) { return z > 0.f && z <= FLT_MAX; }

// Geometry of sequence b; false (and the data flag) when cu_gamma is malformed.
template <bool RAGGED>
__device__ __forceinline__ bool seq_geom(const Args& a, int b, int& base, int& g) {
  if (!RAGGED) {
    base = b * a.gamma;
    g = a.gamma;
    return true;
  }
  const int c0 = a.cu[b], c1 = a.cu[b + 1];
  base = c0;
  g = c1 - c0;
  bool ok = c0 >= 0 && c1 >= c0 && c1 <= a.R && g <= a.max_gamma;
  if (b == 0 && c0 != 0) ok = false;
  if (b == a.B - 1 && c1 != a.R) ok = false;
  return ok;
}

// ============================================================== step 1
// Row statistics of one split of one draft row: m = max l, z = sum exp2((l - m) * k2).
template <typename T, bool ALIGNED, bool RAGGED>
__global__ __launch_bounds__(kThreads) void k_rowstats(Args a) {
  __shared__ float s_m[kWaves], s_z[kWaves];
  const int d = blockIdx.x / a.split, k = blockIdx.x - d * a.split;
  const int b = RAGGED ? seq_of_row(a.cu, a.B, d) : d / a.gamma;
  const T* row = static_cast<const T*>(a.logits) + static_cast<size_t>(d + b) * a.V;
  const int lo = k * a.span, hi = min(a.V, lo + a.span);
  const float k2 = a.k2;
  float m = -FLT_MAX;
  float s[kGroup];
#pragma unroll
  for (int j = 0; j < kGroup; ++j) s[j] = 0.f;

  if (ALIGNED) {
    const int g1 = hi >> 3;
    int g = (lo >> 3) + threadIdx.x;
    for (; g + (kUnroll - 1) * kThreads < g1; g += kUnroll * kThreads) {
      float x[kUnroll][kGroup];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) load_group(row, static_cast<size_t>(g + u * kThreads) * kGroup, x[u]);
      float bm = x[0][0];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int j = 0; j < kGroup; ++j) bm = fmaxf(bm, x[u][j]);
      if (bm > m) {
        const float sc = fast_exp2((m - bm) * k2);
#pragma unroll
        for (int j = 0; j < kGroup; ++j) s[j] *= sc;
        m = bm;
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int j = 0; j < kGroup; ++j) s[j] += fast_exp2((x[u][j] - m) * k2);
    }
    for (; g < g1; g += kThreads) {
      float x[kGroup];
      load_group(row, static_cast<size_t>(g) * kGroup, x);
      float bm = x[0];
#pragma unroll
      for (int j = 1; j < kGroup; ++j) bm = fmaxf(bm, x[j]);
      if (bm > m) {
        const float sc = fast_exp2((m - bm) * k2);
#pragma unroll
        for (int j = 0; j < kGroup; ++j) s[j] *= sc;
        m = bm;
      }
#pragma unroll
      for (int j = 0; j < kGroup; ++j) s[j] += fast_exp2((x[j] - m) * k2);
    }
  } else {
    for (int e = lo + threadIdx.x; e < hi; e += kThreads) {
      const float x = load_one(row, e);
      if (x > m) {
        s[0] *= fast_exp2((m - x) * k2);
        m = x;
      }
      s[0] += fast_exp2((x - m) * k2);
    }
  }
  float z = ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o), z2 = __shfl_xor(z, o);
    lse_merge(m, z, m2, z2, k2);
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    s_m[w] = m;
    s_z[w] = z;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = s_m[0], Z = s_z[0];
    for (int i = 1; i < kWaves; ++i) lse_merge(M, Z, s_m[i], s_z[i], k2);
    a.p1[blockIdx.x] = RowStat{M, Z};
  }
}

// Greedy twin: max raw logit of one split of one draft row and its lowest index.
template <typename T, bool ALIGNED, bool RAGGED>
__global__ __launch_bounds__(kThreads) void k_rowargmax(Args a) {
  __shared__ float s_v[kWaves];
  __shared__ int s_i[kWaves];
  const int d = blockIdx.x / a.split, k = blockIdx.x - d * a.split;
  const int b = RAGGED ? seq_of_row(a.cu, a.B, d) : d / a.gamma;
  const T* row = static_cast<const T*>(a.logits) + static_cast<size_t>(d + b) * a.V;
  const int lo = k * a.span, hi = min(a.V, lo + a.span);
  float bv = -INFINITY;
  int bi = INT_MAX;
  if (ALIGNED) {
    const int g1 = hi >> 3;
    int g = (lo >> 3) + threadIdx.x;
    if (g < g1) bi = g * kGroup;  // seed: a row of -inf still yields its first index
    for (; g + (kUnroll - 1) * kThreads < g1; g += kUnroll * kThreads) {
      float x[kUnroll][kGroup];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) load_group(row, static_cast<size_t>(g + u * kThreads) * kGroup, x[u]);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int j = 0; j < kGroup; ++j)
          if (x[u][j] > bv) {
            bv = x[u][j];
            bi = (g + u * kThreads) * kGroup + j;
          }
    }
    for (; g < g1; g += kThreads) {
      float x[kGroup];
      load_group(row, static_cast<size_t>(g) * kGroup, x);
#pragma unroll
      for (int j = 0; j < kGroup; ++j)
        if (x[j] > bv) {
          bv = x[j];
          bi = g * kGroup + j;
        }
    }
  } else {
    int e = lo + threadIdx.x;
    if (e < hi) bi = e;
    for (; e < hi; e += kThreads) {
      const float x = load_one(row, e);
      if (x > bv) {
        bv = x;
        bi = e;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(bv, o);
    const int i2 = __shfl_xor(bi, o);
    argmax_merge(bv, bi, v2, i2);
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    s_v[w] = bv;
    s_i[w] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float V = s_v[0];
    int I = s_i[0];
    for (int i = 1; i < kWaves; ++i) argmax_merge(V, I, s_v[i], s_i[i]);
    a.p1[blockIdx.x] = RowStat{V, __int_as_float(I)};
  }
}

// ============================================================== step 2 (sampling)
// Load this thread's part of chunk c of a row: groups (tid + k * kThreads), k < 2.
// Entries past V read as `fill`.
template <typename T, bool ALIGNED>
__device__ __forceinline__ void load_chunk(const T* row, int V, int c, float (&x)[kChunkGroups][kGroup], float fill) {
#pragma unroll
  for (int k = 0; k < kChunkGroups; ++k) {
    const int e = c * kChunk + (threadIdx.x + k * kThreads) * kGroup;
    if (ALIGNED) {
      if (e < V) {
        load_group(row, e, x[k]);
      } else {
#pragma unroll
        for (int j = 0; j < kGroup; ++j) x[k][j] = fill;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kGroup; ++j) x[k][j] = (e + j < V) ? load_one(row, e + j) : fill;
    }
  }
}

template <typename T, bool ALIGNED, bool RAGGED>
__global__ __launch_bounds__(kThreads) void k_sample_chunks(Args a) {
  __shared__ int s_n;
  __shared__ float2 s_mz[kMaxGamma];
  __shared__ double s_red[kWaves * 3];
  __shared__ float s_f[kWaves];
  const int b = blockIdx.x / a.nc, c = blockIdx.x - b * a.nc;
  int base, g;
  if (!seq_geom<RAGGED>(a, b, base, g)) {
    if (c == 0 && threadIdx.x == 0) {
      atomicOr(a.err, SV_DATA_CU_GAMMA);
      SeqInfo si{};
      si.mode = MODE_INVALID;
      a.info[b] = si;
      a.acc[b] = -1;
    }
    return;
  }
  if (threadIdx.x == 0) s_n = g;
  __syncthreads();
  const T* L = static_cast<const T*>(a.logits);

  // ---- prologue: accept test of every draft position ([P1] ch.3; [P3] 단계 3)
  for (int i = threadIdx.x; i < g; i += kThreads) {
    const int d = base + i;
    float M = -FLT_MAX, Z = 0.f;
    for (int k = 0; k < a.split; ++k) {
      const RowStat r = a.p1[static_cast<size_t>(d) * a.split + k];
      lse_merge(M, Z, r.m, r.z, a.k2);
    }
    s_mz[i] = make_float2(M, Z);
    const int x = a.ids[d];
    const bool valid = x >= 0 && x < a.V;
    double px = __builtin_nan("");
    bool accept = false;
    if (valid) {
      const float lx = load_one(L, static_cast<size_t>(d + b) * a.V + x);
      px = exp((static_cast<double>(lx) - static_cast<double>(M)) * a.invT) / static_cast<double>(Z);
      const double qx = a.q[static_cast<size_t>(d) * a.V + x];
      const double thr = px >= qx ? 1.0 : px / qx;  // min(1, p/q) without dividing when p >= q
      const float uu = a.u[base + b + i];
      accept = static_cast<double>(uu) < thr;      // strict
      if (c == 0 && !(uu >= 0.f && uu < 1.f)) atomicOr(a.err, SV_DATA_UNIFORM);
    }
    if (!accept) atomicMin(&s_n, i);
    if (c == 0) {
      if (!valid) atomicOr(a.err, SV_DATA_DRAFT_ID);
      if (!(finite_pos(Z) && M <= FLT_MAX)) atomicOr(a.err, SV_DATA_NONFINITE);
      if (a.pdraft) a.pdraft[d] = static_cast<float>(px);
    }
  }
  __syncthreads();
  const int n = s_n;  // first rejection, or g when all accepted ([P1] ch.2)

  if (c == 0) {
    for (int i = threadIdx.x; i < n; i += kThreads) a.emitted[base + b + i] = a.ids[base + i];
    if (threadIdx.x == 0) {
      SeqInfo si{};
      si.n = n;
      si.mode = n < g ? MODE_RESIDUAL : MODE_BONUS;
      si.m = n < g ? s_mz[n].x : 0.f;
      si.z = n < g ? s_mz[n].y : 0.f;
      si.g = g;
      si.base = base;
      a.info[b] = si;
      a.acc[b] = n;
    }
  }

  double acc[3] = {0.0, 0.0, 0.0};
  float mc = -INFINITY;  // bonus: chunk max of the raw logits
  if (n < g) {
    // ---- residual sweep of chunk c of row n ([P1] ch.3 residual; [P3] 단계 3 x')
    const float M = s_mz[n].x;
    const double Zq = static_cast<double>(s_mz[n].y);
    const T* lrow = L + static_cast<size_t>(base + b + n) * a.V;
    const float* qrow = a.q + static_cast<size_t>(base + n) * a.V;
    float lx[kChunkGroups][kGroup], qx[kChunkGroups][kGroup];
    load_chunk<T, ALIGNED>(lrow, a.V, c, lx, -INFINITY);
    load_chunk<float, ALIGNED>(qrow, a.V, c, qx, 0.f);
#pragma unroll
    for (int k = 0; k < kChunkGroups; ++k)
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        const double ev = exp((static_cast<double>(lx[k][j]) - static_cast<double>(M)) * a.invT);
        const double qv = static_cast<double>(qx[k][j]);
        const bool pos = ev > qv * Zq;
        acc[0] += pos ? ev : 0.0;
        acc[1] += pos ? qv : 0.0;
        acc[2] += ev;
      }
  } else {
    // ---- bonus sweep of chunk c of row g ([P1] ch.2 bonus; [P3] 단계 3)
    const T* lrow = L + static_cast<size_t>(base + b + g) * a.V;
    float lx[kChunkGroups][kGroup];
    load_chunk<T, ALIGNED>(lrow, a.V, c, lx, -INFINITY);
#pragma unroll
    for (int k = 0; k < kChunkGroups; ++k)
#pragma unroll
      for (int j = 0; j < kGroup; ++j) mc = fmaxf(mc, lx[k][j]);
    mc = block_max(mc, s_f);
    if (mc > -INFINITY) {
#pragma unroll
      for (int k = 0; k < kChunkGroups; ++k)
#pragma unroll
        for (int j = 0; j < kGroup; ++j)
          acc[1] += exp((static_cast<double>(lx[k][j]) - static_cast<double>(mc)) * a.invT);
    }
  }
  block_sum<3>(acc, s_red);
  if (threadIdx.x == 0) {
    double* o = a.csum + (static_cast<size_t>(b) * a.nc + c) * 3;
    o[0] = n < g ? acc[0] : static_cast<double>(mc);
    o[1] = acc[1];
    o[2] = acc[2];
  }
}

// ============================================================== step 3 (sampling)
template <typename T, bool ALIGNED, bool RAGGED>
__global__ __launch_bounds__(kThreads) void k_sample_finalize(Args a) {
  __shared__ double s_d[kWaves];
  __shared__ int s_i[kWaves];
  const int b = blockIdx.x;
  const SeqInfo si = a.info[b];
  if (si.mode == MODE_INVALID) return;
  const int n = si.n, g = si.g, base = si.base;
  const float uf = a.u[base + b + g];
  const double u = uf;
  const double* cs = a.csum + static_cast<size_t>(b) * a.nc * 3;
  const int nc = a.nc;

  // kind 0: residual max(0, p - q); 1: degenerate residual, draw from p; 2: bonus from p
  int kind;
  double Zs = 0.0, S = 0.0, invZ = 0.0, Mb = -INFINITY, t;
  if (si.mode == MODE_RESIDUAL) {
    for (int c = 0; c < nc; ++c) Zs += cs[c * 3 + 2];
    invZ = 1.0 / Zs;
    for (int c = 0; c < nc; ++c) S += cs[c * 3 + 0] * invZ - cs[c * 3 + 1];
    if (S > 0.0) {
      kind = 0;
      t = u * S;
    } else {
      kind = 1;
      t = u * Zs;
    }
  } else {
    for (int c = 0; c < nc; ++c) Mb = fmax(Mb, cs[c * 3 + 0]);
    for (int c = 0; c < nc; ++c) {
      const double mc = cs[c * 3 + 0];
      if (mc > -INFINITY) Zs += cs[c * 3 + 1] * exp((mc - Mb) * a.invT);
    }
    kind = 2;
    t = u * Zs;
  }
  if (threadIdx.x == 0) {
    if (!(Zs > 0.0 && Zs <= DBL_MAX)) atomicOr(a.err, SV_DATA_NONFINITE);
    if (!(uf >= 0.f && uf < 1.f)) atomicOr(a.err, SV_DATA_UNIFORM);
  }
  auto weight = [&](int c) -> double {
    if (kind == 0) return cs[c * 3 + 0] * invZ - cs[c * 3 + 1];
    if (kind == 1) return cs[c * 3 + 2];
    const double mc = cs[c * 3 + 0];
    return mc > -INFINITY ? cs[c * 3 + 1] * exp((mc - Mb) * a.invT) : 0.0;
  };
  // chunk where the inclusive prefix first exceeds t
  double P = 0.0;
  int cstar = -1;
  for (int c = 0; c < nc; ++c) {
    const double w = weight(c);
    if (P + w > t) {
      cstar = c;
      break;
    }
    P += w;
  }
  bool take_last = false;
  if (cstar < 0) {  // no crossing (rounding, or u >= 1): last positive-weight token
    take_last = true;
    for (int c = nc - 1; c >= 0; --c)
      if (weight(c) > 0.0) {
        cstar = c;
        break;
      }
  }
  int tok = a.V - 1;
  if (cstar >= 0) {
    const T* L = static_cast<const T*>(a.logits);
    const int row_off = kind == 2 ? g : n;
    const T* lrow = L + static_cast<size_t>(base + b + row_off) * a.V;
    const int e0 = cstar * kChunk + threadIdx.x * (kGroup * kChunkGroups);
    float lx[kChunkGroups][kGroup], qx[kChunkGroups][kGroup];
#pragma unroll
    for (int k = 0; k < kChunkGroups; ++k) {
      const int e = e0 + k * kGroup;
      if (ALIGNED && e < a.V) {
        load_group(lrow, e, lx[k]);
      } else {
#pragma unroll
        for (int j = 0; j < kGroup; ++j) lx[k][j] = (e + j < a.V) ? load_one(lrow, e + j) : -INFINITY;
      }
    }
    if (kind == 0) {
      const float* qrow = a.q + static_cast<size_t>(base + n) * a.V;
#pragma unroll
      for (int k = 0; k < kChunkGroups; ++k) {
        const int e = e0 + k * kGroup;
        if (ALIGNED && e < a.V) {
          load_group(qrow, e, qx[k]);
        } else {
#pragma unroll
          for (int j = 0; j < kGroup; ++j) qx[k][j] = (e + j < a.V) ? qrow[e + j] : 0.f;
        }
      }
    }
    const double ref = kind == 2 ? Mb : static_cast<double>(si.m);
    const double Zq = static_cast<double>(si.z);
    double r[kChunkGroups * kGroup];
    double tot = 0.0;
#pragma unroll
    for (int k = 0; k < kChunkGroups; ++k)
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        const double ev = exp((static_cast<double>(lx[k][j]) - ref) * a.invT);
        double w = ev;
        if (kind == 0) {
          const double qv = static_cast<double>(qx[k][j]);
          w = ev > qv * Zq ? ev * invZ - qv : 0.0;
        }
        r[k * kGroup + j] = w;
        tot += w;
      }
    double run = P + block_excl_scan(tot, s_d);
    int cand = INT_MAX, lastpos = -1;
#pragma unroll
    for (int j = 0; j < kChunkGroups * kGroup; ++j) {
      run += r[j];
      if (!take_last && cand == INT_MAX && run > t) cand = e0 + j;
      if (r[j] > 0.0) lastpos = e0 + j;
    }
    cand = block_min_int(cand, s_i);
    lastpos = block_max_int(lastpos, s_i);
    tok = cand != INT_MAX ? cand : (lastpos >= 0 ? lastpos : a.V - 1);
  }
  if (threadIdx.x == 0) {
    a.emitted[base + b + n] = tok;
    a.rsum[b] = kind == 2 ? 0.f : static_cast<float>(S);
  }
  for (int i = n + 1 + threadIdx.x; i <= g; i += kThreads) a.emitted[base + b + i] = -1;
}

// ============================================================== steps 2-3 (greedy)
template <typename T, bool ALIGNED, bool RAGGED>
__global__ __launch_bounds__(kThreads) void k_greedy_chunks(Args a) {
  __shared__ int s_n;
  __shared__ int s_tok[kMaxGamma];
  __shared__ float s_v[kWaves];
  __shared__ int s_i[kWaves];
  const int b = blockIdx.x / a.nc, c = blockIdx.x - b * a.nc;
  int base, g;
  if (!seq_geom<RAGGED>(a, b, base, g)) {
    if (c == 0 && threadIdx.x == 0) {
      atomicOr(a.err, SV_DATA_CU_GAMMA);
      SeqInfo si{};
      si.mode = MODE_INVALID;
      a.info[b] = si;
      a.acc[b] = -1;
    }
    return;
  }
  if (threadIdx.x == 0) s_n = g;
  __syncthreads();
  // accept iff the draft equals the target argmax ([P1] ch.3 greedy; [P4])
  for (int i = threadIdx.x; i < g; i += kThreads) {
    const int d = base + i;
    float V = -INFINITY;
    int I = INT_MAX;
    for (int k = 0; k < a.split; ++k) {
      const RowStat r = a.p1[static_cast<size_t>(d) * a.split + k];
      argmax_merge(V, I, r.m, __float_as_int(r.z));
    }
    s_tok[i] = I;
    const int x = a.ids[d];
    if (x != I) atomicMin(&s_n, i);
    if (c == 0 && !(x >= 0 && x < a.V)) atomicOr(a.err, SV_DATA_DRAFT_ID);
  }
  __syncthreads();
  const int n = s_n;
  if (c == 0) {
    for (int i = threadIdx.x; i < n; i += kThreads) a.emitted[base + b + i] = a.ids[base + i];
    if (threadIdx.x == 0) {
      SeqInfo si{};
      si.n = n;
      si.mode = MODE_GREEDY;
      si.tok = n < g ? s_tok[n] : -1;
      si.g = g;
      si.base = base;
      a.info[b] = si;
      a.acc[b] = n;
    }
  }
  if (n < g) return;  // the bonus row is read only when every draft was accepted
  const T* lrow = static_cast<const T*>(a.logits) + static_cast<size_t>(base + b + g) * a.V;
  float lx[kChunkGroups][kGroup];
  load_chunk<T, ALIGNED>(lrow, a.V, c, lx, -INFINITY);
  float bv = -INFINITY;
  int bi = INT_MAX;
#pragma unroll
  for (int k = 0; k < kChunkGroups; ++k) {
    const int e = c * kChunk + (threadIdx.x + k * kThreads) * kGroup;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      if (e + j < a.V && bi == INT_MAX) bi = e + j;  // seed with the first in-range entry
      if (lx[k][j] > bv) {
        bv = lx[k][j];
        bi = e + j;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(bv, o);
    const int i2 = __shfl_xor(bi, o);
    argmax_merge(bv, bi, v2, i2);
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    s_v[w] = bv;
    s_i[w] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float V = s_v[0];
    int I = s_i[0];
    for (int i = 1; i < kWaves; ++i) argmax_merge(V, I, s_v[i], s_i[i]);
    double* o = a.csum + (static_cast<size_t>(b) * a.nc + c) * 3;
    o[0] = V;
    o[1] = static_cast<double>(I);
  }
}

__global__ __launch_bounds__(64) void k_greedy_finalize(Args a) {
  const int b = blockIdx.x;
  const SeqInfo si = a.info[b];
  if (si.mode == MODE_INVALID) return;
  const int n = si.n, g = si.g, base = si.base;
  int tok = si.tok;
  if (n == g) {
    const double* cs = a.csum + static_cast<size_t>(b) * a.nc * 3;
    float V = -INFINITY;
    int I = INT_MAX;
    for (int c = 0; c < a.nc; ++c) argmax_merge(V, I, static_cast<float>(cs[c * 3]), static_cast<int>(cs[c * 3 + 1]));
    tok = I;
  }
  if (threadIdx.x == 0) {
    a.emitted[base + b + n] = tok;
    a.rsum[b] = 0.f;
  }
  for (int i = n + 1 + threadIdx.x; i <= g; i += 64) a.emitted[base + b + i] = -1;
}

// ============================================================== host side
const char* kKernelNames[2][3] = {
    {"k_rowstats", "k_sample_chunks", "k_sample_finalize"},
    {"k_rowargmax", "k_greedy_chunks", "k_greedy_finalize"},
};

}  // namespace

struct spec_verify_ctx {
  int device = 0, V = 0, dtype = 0, max_batch = 0, max_rows = 0, max_gamma = 0, nc = 0, cus = 0;
  void* ws = nullptr;
  RowStat* p1 = nullptr;
  double* csum = nullptr;
  SeqInfo* info = nullptr;
  int* err = nullptr;
  hipStream_t last_stream = nullptr;
  bool ran = false;
  // measurement: kKernels + 1 events per recorded run, for up to timing_cap runs
  int timing_cap = 0, timing_runs = 0;
  hipEvent_t* ev = nullptr;
  int nk = 0;
  const char* kname[3] = {nullptr, nullptr, nullptr};
  char msg[512] = {0};
};

namespace {

void set_msg(char* dst, int cap, const char* s) {
  if (!dst || cap <= 0) return;
  snprintf(dst, static_cast<size_t>(cap), "%s", s);
}

int hip_fail(spec_verify_ctx* ctx, const char* what, hipError_t e) {
  if (ctx) snprintf(ctx->msg, sizeof(ctx->msg), "%s: %s", what, hipGetErrorString(e));
  return SV_EHIP;
}

// Restores the calling thread's current device on scope exit.
struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

constexpr int kKernels = 3;

template <typename T, bool AL, bool RG>
hipError_t launch_path(spec_verify_ctx* ctx, const Args& a, hipStream_t st, bool greedy) {
  const dim3 blk(kThreads);
  const bool rec = ctx->timing_runs < ctx->timing_cap;
  hipEvent_t* ev = rec ? ctx->ev + static_cast<size_t>(ctx->timing_runs) * (kKernels + 1) : nullptr;
  auto mark = [&](int i) {
    if (ev) (void)hipEventRecord(ev[i], st);
  };
  mark(0);
  if (a.R > 0) {
    const dim3 grid(static_cast<unsigned>(a.R) * a.split);
    if (greedy)
      hipLaunchKernelGGL((k_rowargmax<T, AL, RG>), grid, blk, 0, st, a);
    else
      hipLaunchKernelGGL((k_rowstats<T, AL, RG>), grid, blk, 0, st, a);
  }
  mark(1);
  const dim3 grid2(static_cast<unsigned>(a.B) * a.nc);
  if (greedy)
    hipLaunchKernelGGL((k_greedy_chunks<T, AL, RG>), grid2, blk, 0, st, a);
  else
    hipLaunchKernelGGL((k_sample_chunks<T, AL, RG>), grid2, blk, 0, st, a);
  mark(2);
  if (greedy)
    hipLaunchKernelGGL(k_greedy_finalize, dim3(a.B), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((k_sample_finalize<T, AL, RG>), dim3(a.B), blk, 0, st, a);
  mark(3);
  if (rec) ++ctx->timing_runs;
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dt(spec_verify_ctx* ctx, const Args& a, hipStream_t st, bool greedy, bool aligned, bool ragged) {
  if (aligned)
    return ragged ? launch_path<T, true, true>(ctx, a, st, greedy) : launch_path<T, true, false>(ctx, a, st, greedy);
  return ragged ? launch_path<T, false, true>(ctx, a, st, greedy) : launch_path<T, false, false>(ctx, a, st, greedy);
}

void free_events(spec_verify_ctx* ctx) {
  if (ctx->ev) {
    const size_t n = static_cast<size_t>(ctx->timing_cap) * (kKernels + 1);
    for (size_t i = 0; i < n; ++i)
      if (ctx->ev[i]) (void)hipEventDestroy(ctx->ev[i]);
    delete[] ctx->ev;
  }
  ctx->ev = nullptr;
  ctx->timing_cap = ctx->timing_runs = 0;
}

// Row-stats split: aim for >= 2048 workgroups, >= 2048 entries per split.
void choose_split(int R, int V, int& split, int& span) {
  int s = R > 0 ? (2048 + R - 1) / R : 1;
  s = s < 1 ? 1 : (s > kMaxSplit ? kMaxSplit : s);
  const int by_len = (V + 2047) / 2048;
  if (s > by_len) s = by_len < 1 ? 1 : by_len;
  int sp = (V + s - 1) / s;
  sp = (sp + kGroup - 1) / kGroup * kGroup;
  split = (V + sp - 1) / sp;
  span = sp;
}

}  // namespace

extern "C" {

int spec_verify_check_args(int vocab, int logits_dtype, int max_batch, int max_draft_rows, int max_gamma,
                           int batch, int gamma, int has_cu_gamma, int total_draft_rows, float temperature,
                           int has_logits, int has_q, int has_draft_ids, int has_uniforms,
                           int has_accepted_count, int has_emitted_tokens, int has_residual_sum, char* msg,
                           int msg_cap) {
  auto bad = [&](const char* s) {
    set_msg(msg, msg_cap, s);
    return SV_EINVAL;
  };
  if (vocab < 1) return bad("vocab must be >= 1");
  if (logits_dtype != SV_F32 && logits_dtype != SV_BF16) return bad("logits_dtype must be SV_F32 or SV_BF16");
  if (batch < 0) return bad("batch must be >= 0");
  if (batch > max_batch) return bad("batch exceeds max_batch");
  if (total_draft_rows < 0) return bad("total_draft_rows must be >= 0");
  if (total_draft_rows > max_draft_rows) return bad("total_draft_rows exceeds max_draft_rows");
  if (has_cu_gamma) {
    if (gamma != -1) return bad("gamma must be -1 when cu_gamma is given");
  } else {
    if (gamma < 0) return bad("gamma must be >= 0 without cu_gamma");
    if (gamma > max_gamma) return bad("gamma exceeds max_gamma");
    if (static_cast<long long>(batch) * gamma != total_draft_rows)
      return bad("total_draft_rows must equal batch * gamma");
  }
  if (!(temperature >= 0.f) || !(temperature <= FLT_MAX)) return bad("temperature must be finite and >= 0");
  if (batch == 0) {
    set_msg(msg, msg_cap, "");
    return SV_OK;
  }
  if (!has_logits) return bad("logits is NULL");
  if (total_draft_rows > 0 && !has_draft_ids) return bad("draft_ids is NULL");
  if (temperature > 0.f) {
    if (!has_uniforms) return bad("uniforms is NULL with T > 0");
    if (total_draft_rows > 0 && !has_q) return bad("q is NULL with T > 0");
  }
  if (!has_accepted_count || !has_emitted_tokens || !has_residual_sum) return bad("an output pointer is NULL");
  set_msg(msg, msg_cap, "");
  return SV_OK;
}

int spec_verify_create(spec_verify_ctx** out, int device, int vocab, int logits_dtype, int max_batch,
                       int max_draft_rows, int max_gamma) {
  if (!out) return SV_EINVAL;
  *out = nullptr;
  if (vocab < 1 || max_batch < 0 || max_draft_rows < 0 || max_gamma < 0 || max_gamma > kMaxGamma ||
      max_batch > kMaxBatch || (logits_dtype != SV_F32 && logits_dtype != SV_BF16))
    return SV_EINVAL;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) return SV_EHIP;
  DeviceGuard guard(device);
  spec_verify_ctx* ctx = new (std::nothrow) spec_verify_ctx();
  if (!ctx) return SV_ENOMEM;
  ctx->device = device;
  ctx->V = vocab;
  ctx->dtype = logits_dtype;
  ctx->max_batch = max_batch;
  ctx->max_rows = max_draft_rows;
  ctx->max_gamma = max_gamma;
  ctx->nc = (vocab + kChunk - 1) / kChunk;
  if (hipDeviceGetAttribute(&ctx->cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) ctx->cus = 256;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const int max_split = (vocab + 2047) / 2048 < kMaxSplit ? (vocab + 2047) / 2048 : kMaxSplit;
  const size_t n_p1 =
      up(sizeof(RowStat) * static_cast<size_t>(max_draft_rows > 0 ? max_draft_rows : 1) * max_split);
  const size_t n_cs = up(sizeof(double) * 3 * static_cast<size_t>(max_batch > 0 ? max_batch : 1) * ctx->nc);
  const size_t n_in = up(sizeof(SeqInfo) * static_cast<size_t>(max_batch > 0 ? max_batch : 1));
  const size_t n_er = 256;
  if (hipMalloc(&ctx->ws, n_p1 + n_cs + n_in + n_er) != hipSuccess) {
    delete ctx;
    return SV_ENOMEM;
  }
  char* p = static_cast<char*>(ctx->ws);
  ctx->p1 = reinterpret_cast<RowStat*>(p);
  ctx->csum = reinterpret_cast<double*>(p + n_p1);
  ctx->info = reinterpret_cast<SeqInfo*>(p + n_p1 + n_cs);
  ctx->err = reinterpret_cast<int*>(p + n_p1 + n_cs + n_in);
  if (hipMemset(ctx->err, 0, n_er) != hipSuccess) {
    (void)hipFree(ctx->ws);
    delete ctx;
    return SV_EHIP;
  }
  *out = ctx;
  return SV_OK;
}

int spec_verify_run(spec_verify_ctx* ctx, void* hip_stream, int batch, int gamma, const int32_t* cu_gamma,
                    int total_draft_rows, float temperature, const void* logits, const float* q,
                    const int32_t* draft_ids, const float* uniforms, int32_t* accepted_count,
                    int32_t* emitted_tokens, float* residual_sum, float* p_draft) {
  if (!ctx) return SV_EINVAL;
  const int rc = spec_verify_check_args(
      ctx->V, ctx->dtype, ctx->max_batch, ctx->max_rows, ctx->max_gamma, batch, gamma, cu_gamma != nullptr,
      total_draft_rows, temperature, logits != nullptr, q != nullptr, draft_ids != nullptr, uniforms != nullptr,
      accepted_count != nullptr, emitted_tokens != nullptr, residual_sum != nullptr, ctx->msg, sizeof(ctx->msg));
  if (rc != SV_OK) return rc;
  if (batch == 0) return SV_OK;
  const size_t esz = ctx->dtype == SV_BF16 ? 2 : 4;
  if (reinterpret_cast<uintptr_t>(logits) % esz != 0 || (q && reinterpret_cast<uintptr_t>(q) % 4 != 0)) {
    set_msg(ctx->msg, sizeof(ctx->msg), "logits / q not aligned to their element size");
    return SV_EINVAL;
  }
  if (cu_gamma && batch > kMaxRaggedBatch) {
    set_msg(ctx->msg, sizeof(ctx->msg), "ragged batches (cu_gamma) are limited to 65536 sequences");
    return SV_EINVAL;
  }
  const bool greedy = temperature == 0.f;
  const bool aligned = ctx->V % kGroup == 0 && reinterpret_cast<uintptr_t>(logits) % 16 == 0 &&
                       (greedy || reinterpret_cast<uintptr_t>(q) % 16 == 0);
  Args a{};
  a.logits = logits;
  a.q = greedy ? nullptr : q;
  a.ids = draft_ids;
  a.u = greedy ? nullptr : uniforms;
  a.cu = cu_gamma;
  a.acc = accepted_count;
  a.emitted = emitted_tokens;
  a.rsum = residual_sum;
  a.pdraft = greedy ? nullptr : p_draft;
  a.p1 = ctx->p1;
  a.csum = ctx->csum;
  a.info = ctx->info;
  a.err = ctx->err;
  a.B = batch;
  a.gamma = cu_gamma ? -1 : gamma;
  a.V = ctx->V;
  a.R = total_draft_rows;
  a.nc = ctx->nc;
  a.max_gamma = ctx->max_gamma;
  choose_split(a.R, a.V, a.split, a.span);
  const unsigned long long max_threads = 1ull << 32;
  if (static_cast<unsigned long long>(a.R) * a.split * kThreads >= max_threads ||
      static_cast<unsigned long long>(a.B) * a.nc * kThreads >= max_threads) {
    set_msg(ctx->msg, sizeof(ctx->msg), "launch grid too large: reduce the batch");
    return SV_EINVAL;
  }
  if (greedy) {
    a.k2 = 0.f;
    a.invT = 0.0;
  } else {
    a.invT = 1.0 / static_cast<double>(temperature);
    a.k2 = static_cast<float>(1.4426950408889634 * a.invT);
  }
  DeviceGuard guard(ctx->device);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const hipError_t e = ctx->dtype == SV_BF16
                           ? launch_dt<uint16_t>(ctx, a, st, greedy, aligned, cu_gamma != nullptr)
                           : launch_dt<float>(ctx, a, st, greedy, aligned, cu_gamma != nullptr);
  if (e != hipSuccess) return hip_fail(ctx, "kernel launch", e);
  ctx->last_stream = st;
  ctx->ran = true;
  ctx->nk = kKernels;
  for (int i = 0; i < kKernels; ++i) ctx->kname[i] = kKernelNames[greedy ? 1 : 0][i];
  return SV_OK;
}

int spec_verify_status(spec_verify_ctx* ctx) {
  if (!ctx) return SV_EINVAL;
  DeviceGuard guard(ctx->device);
  hipError_t e = ctx->ran ? hipStreamSynchronize(ctx->last_stream) : hipSuccess;
  if (e != hipSuccess) return hip_fail(ctx, "hipStreamSynchronize", e);
  int flag = 0;
  e = hipMemcpy(&flag, ctx->err, sizeof(int), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(ctx, "hipMemcpy", e);
  if (flag == 0) return SV_OK;
  const int zero = 0;
  e = hipMemcpy(ctx->err, &zero, sizeof(int), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(ctx, "hipMemcpy", e);
  snprintf(ctx->msg, sizeof(ctx->msg), "device data error flags 0x%x:%s%s%s%s", flag,
           (flag & SV_DATA_DRAFT_ID) ? " draft-id-out-of-range" : "",
           (flag & SV_DATA_NONFINITE) ? " non-finite-normaliser" : "",
           (flag & SV_DATA_UNIFORM) ? " uniform-out-of-[0,1)" : "",
           (flag & SV_DATA_CU_GAMMA) ? " malformed-cu_gamma" : "");
  return SV_EDATA;
}

const char* spec_verify_last_error(const spec_verify_ctx* ctx) { return ctx ? ctx->msg : ""; }

void spec_verify_destroy(spec_verify_ctx* ctx) {
  if (!ctx) return;
  {
    DeviceGuard guard(ctx->device);
    (void)hipDeviceSynchronize();
    free_events(ctx);
    if (ctx->ws) (void)hipFree(ctx->ws);
  }
  delete ctx;
}

int spec_verify_set_timing(spec_verify_ctx* ctx, int runs) {
  if (!ctx || runs < 0) return SV_EINVAL;
  DeviceGuard guard(ctx->device);
  (void)hipDeviceSynchronize();
  free_events(ctx);
  if (runs == 0) return SV_OK;
  const size_t n = static_cast<size_t>(runs) * (kKernels + 1);
  ctx->ev = new (std::nothrow) hipEvent_t[n]();
  if (!ctx->ev) return SV_ENOMEM;
  ctx->timing_cap = runs;
  for (size_t i = 0; i < n; ++i) {
    const hipError_t e = hipEventCreate(&ctx->ev[i]);
    if (e != hipSuccess) {
      free_events(ctx);
      return hip_fail(ctx, "hipEventCreate", e);
    }
  }
  ctx->timing_runs = 0;
  return SV_OK;
}

int spec_verify_kernel_times(spec_verify_ctx* ctx, float* ms, const char** names, int cap, int* runs) {
  if (!ctx) return -SV_EINVAL;
  if (runs) *runs = ctx->timing_runs;
  if (ctx->timing_runs == 0) return 0;
  DeviceGuard guard(ctx->device);
  const int R = ctx->timing_runs;
  hipError_t e = hipEventSynchronize(ctx->ev[static_cast<size_t>(R) * (kKernels + 1) - 1]);
  if (e != hipSuccess) return -hip_fail(ctx, "hipEventSynchronize", e);
  for (int k = 0; k < ctx->nk && k < cap; ++k) {
    double sum = 0.0;
    for (int r = 0; r < R; ++r) {
      float t = 0.f;
      hipEvent_t* ev = ctx->ev + static_cast<size_t>(r) * (kKernels + 1);
      e = hipEventElapsedTime(&t, ev[k], ev[k + 1]);
      if (e != hipSuccess) return -hip_fail(ctx, "hipEventElapsedTime", e);
      sum += t;
    }
    if (ms) ms[k] = static_cast<float>(sum / R);
    if (names) names[k] = ctx->kname[k];
  }
  ctx->timing_runs = 0;  // the next runs record afresh
  return ctx->nk;
}

}  // extern "C"

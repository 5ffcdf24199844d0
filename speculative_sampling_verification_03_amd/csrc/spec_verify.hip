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
// Launch plans (all on the caller's stream, no host sync):
//   * one launch (k_verify_seq; greedy: k_greedy_seq1), B >= 0.55 (greedy: 0.8) times
//     the compute units: one 1024-thread workgroup per sequence judges its draft rows
//     left to right in one read each (base-2 online max and sum in fp32, the accept
//     test in fp64), stops at the first rejection and draws from the one row it
//     needs. A ragged batch first orders its sequences longest first
//     (k_order_by_gamma). Greedy batches of up to four times the compute units add
//     helper workgroups (k_greedy_help).
//   * two launches, smaller batches: k_rowstats / k_rowargmax, grid = (draft rows) x
//     split, 256 threads, one read of every draft row, keep each split's (c, z) or
//     (max, index); then k_sample_seq / k_greedy_seq, one workgroup per sequence, find
//     the first rejection and draw; with at most half as many sequences as compute units
//     k_draw_part shares each draw over two or four workgroups, the last to finish
//     completing it.
//   * one launch for small sampling batches (k_verify_group), B below the compute units:
//     B x gamma x split 256-thread workgroups, all resident at once, read every draft row
//     in parallel chunks; the workgroups of a sequence wait for each other's pass-1
//     records, reach the same first rejection and sweep the drawn row together, the
//     wave of the first unit completing the draw. Rows of at most 4096 entries take one
//     workgroup per sequence instead (k_verify_tiny), its waves handing over through LDS.
//   * rows with no drafts (k_sample_rows, k_sample_weights): one token per row.
//   * vocabulary shards (k_vs_rows, k_vs_decide, k_vs_finish): one device's part when
//     the columns are split over devices.
// The draw is one fp64 sweep of the drawn row, e(v) = 2^(l(v) k2 - c), exact to
// 1.5e-13 relative (bf16 rows through an LDS value table, fp32 rows through exp2_tab),
// with normalisation deferred: with Z32 from pass 1, w(v) = e(v) - q(v) Z32, and a
// region keeps D = sum max(w, 0), Q = sum_{w > 0} q, Zr = sum e. Since
// e/Z64 - q = w/Z64 - q (Z64 - Z32)/Z64, the region's residual mass is
// D/Z64 - Q (Z64 - Z32)/Z64 with Z64 = sum Zr. The region where the prefix crosses
// t = u S is re-swept with an fp64 block scan and the first token whose inclusive
// prefix exceeds t is emitted. The bonus sweep keeps a running region max instead.
//
// Work handed between workgroups of one launch is stored and loaded at system scope,
// past the per-XCD L2 caches, which are not coherent for plain stores. A workgroup waits
// for another only in the small-batch plan, whose grid is resident at once, and every
// such wait is bounded.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <math.h>
#include <stdio.h>
#include <stdint.h>
#include <string.h>

#include <climits>
#include <mutex>
#include <new>

#include "spec_verify.h"
#include "sv_device.h"
#include "sv_adapt.h"
#include "sv_ngram.h"

using namespace sv;

namespace {

// Tuning defaults (compile-time; -D overrides exist for sweeps).
#ifndef SV_UNROLL
#define SV_UNROLL 4
#endif
#ifndef SV_SPLIT_TARGET
#define SV_SPLIT_TARGET 1024
#endif
#ifndef SV_SPLIT_MIN_SPAN
#define SV_SPLIT_MIN_SPAN 2048
#endif
#ifndef SV_GREEDY_HELP
#define SV_GREEDY_HELP 1
#endif
#ifndef SV_GREEDY_WAVES
#define SV_GREEDY_WAVES 3  // owners, then this many - 1 waves of helpers
#endif
constexpr int kMaxSplit = 16;
constexpr int kMaxGamma = 1024;
constexpr int kMaxRaggedBatch = 65536;  // row -> sequence search limit
constexpr int kMaxBatch = 1 << 24;
constexpr int kMaxVocab = 1 << 24;
constexpr int kUnroll = SV_UNROLL;      // groups in flight per thread in the row-stats loop

// Row statistics of one split. Sampling: c = max(l) * k2 (clamped to fp32 range) and
// z = sum 2^(l * k2 - c). Greedy: c = max(l), z = bits of its lowest index.
struct RowStat { float c; float z; };

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
  RowStat* p1;     // [rows][split]
  int32_t* accept; // [rows] decisions of step 1 (rows that are not split)
  float2* lxq;     // [rows] split rows: the draft's logit and q entry, from the split holding it
  int* err;
  int B, gamma, V, R, split, span, max_gamma;
  float k2;        // log2(e) / T, fp32
  double k2d;      // log2(e) / T, fp64
  double kr;       // k2d / k2: scales a pass-1 reference into the fp64 draws (draw_ref)
  // bf16 value table of the one-launch path: magnitudes (bit patterns without the sign)
  // tlo..thi, thi < 0x7F80; tlo > thi when the table is not used
  int tlo, thi;
  int onehot;      // drafts are deterministic: q = one-hot(draft), q is not read
  int nodraft;     // an id of -1 marks "no draft here": rejected without the data flag
  // split draw of the two-launch plan: nslice workgroups sweep one drawn row
  int nslice;
  double* dsum;    // [B][kMaxSub][3] sub-region sums
  int* dcnt;       // [B] slices of the sequence's sweep done (zero between calls)
  // one-launch plan of a ragged batch: the sequence each workgroup takes (null: its index)
  int* order;      // [B]
  // greedy rows with helpers: per sequence, the next row to claim and the participants,
  // each tagged with the call's epoch in the high half, and the first mismatch found,
  // (row << 32) | token
  unsigned long long* gclaim;  // [B]
  unsigned long long* gpart;   // [B]
  unsigned long long* gbest;   // [B]
  unsigned int gepoch;
  // small-batch one-launch plan
  unsigned long long* pchunk;  // [workgroups][4] pass-1 records of the row chunks, tagged
  unsigned long long* psum;    // [B][64][6] unit sums of the drawn rows, tagged
  int uw, nunits;              // unit width (entries) and units of a drawn row
  unsigned ptag;               // this call's tag (nonzero)
};

__device__ __forceinline__ bool finite_pos(float z) { return z > 0.f && z <= FLT_MAX; }
__device__ __forceinline__ bool finite_f(float v) { return v >= -FLT_MAX && v <= FLT_MAX; }
// A draft id that raises the data flag: outside [0, V), unless it is the no-draft mark.
__device__ __forceinline__ bool bad_id(const Args& a, int x) {
  return !(x >= 0 && x < a.V) && !(a.nodraft && x == -1);
}

// Geometry of sequence b; false when cu_gamma is malformed.
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

// Merge (c, z) partial softmax states kept in base 2 (a state stands for z 2^c) that were
// taken with a running max: c is the scaled max of the partial's entries, so z is at
// most the number of terms, the result cannot overflow, and a term that underflows is
// below 2^(C - 126), negligible beside the row's largest entry (which some partial
// counts in full).
__device__ __forceinline__ void lse2_merge(float& c, float& z, float c2, float z2) {
  const float C = fmaxf(c, c2);
  z = z * fast_exp2(c - C) + z2 * fast_exp2(c2 - C);
  c = C;
}

// Pass 1 of the one-launch plan moves a wave's exp2 reference up when an entry lies more
// than this many octaves above it.
constexpr float kRebaseOctaves = 8.f;

// Merge of the states (c, z) held by the 16 lanes of each row of the wave (the wave
// partials of one row). Each z is split as m 2^e (m in [0.5, 1)) and e goes into the
// power of two: C is the largest c + e, Z = sum m 2^(c - C + e) is 0 or lies in
// [0.5, 16], a term that underflows is below 2^-126 of Z, and only the differences
// c - C are rounded, never the references. So the merge loses no partial whatever its
// z: pass 1 keeps z below 2^21, but a partial held against a reference far below its
// largest entry (z near 2^128) would merge as exactly. DPP steps inside the row (a max,
// then a sum): one exp2 per lane and no LDS permutes. Returns row 0's (C, Z),
// wave-uniform; every wave that runs it on the same states gets the same bits.
__device__ __forceinline__ void merge_row16(float c, float z, float& C, float& Z) {
  const float e = static_cast<float>(__builtin_amdgcn_frexp_expf(z));
  int r = __float_as_int(c + e);
  r = __float_as_int(fmaxf(__int_as_float(r), __int_as_float(__builtin_amdgcn_update_dpp(r, r, 0xB1, 0xF, 0xF, false))));
  r = __float_as_int(fmaxf(__int_as_float(r), __int_as_float(__builtin_amdgcn_update_dpp(r, r, 0x4E, 0xF, 0xF, false))));
  r = __float_as_int(fmaxf(__int_as_float(r), __int_as_float(__builtin_amdgcn_update_dpp(r, r, 0x141, 0xF, 0xF, false))));
  r = __float_as_int(fmaxf(__int_as_float(r), __int_as_float(__builtin_amdgcn_update_dpp(r, r, 0x140, 0xF, 0xF, false))));
  C = __int_as_float(__builtin_amdgcn_readlane(r, 0));
  int t = __float_as_int(__builtin_amdgcn_frexp_mantf(z) * fast_exp2((c - C) + e));
  t = __float_as_int(__int_as_float(t) + __int_as_float(__builtin_amdgcn_update_dpp(t, t, 0xB1, 0xF, 0xF, false)));
  t = __float_as_int(__int_as_float(t) + __int_as_float(__builtin_amdgcn_update_dpp(t, t, 0x4E, 0xF, 0xF, false)));
  t = __float_as_int(__int_as_float(t) + __int_as_float(__builtin_amdgcn_update_dpp(t, t, 0x141, 0xF, 0xF, false)));
  t = __float_as_int(__int_as_float(t) + __int_as_float(__builtin_amdgcn_update_dpp(t, t, 0x140, 0xF, 0xF, false)));
  Z = __int_as_float(__builtin_amdgcn_readlane(t, 0));
}

// Accept test of one draft position ([P1] ch.3; [P2] "품질은 rejection sampling이
// 지킨다"; [P3] 단계 3): p(x) = 2^(l_x k2 - c) / z in fp64 (the same normaliser as
// the row statistics), thr = 1 if p(x) >= q(x) else p(x) / q(x), accept iff u < thr.
// An id outside [0, V) rejects; data errors raise the sticky flag.
__device__ __forceinline__ bool accept_decision(int x, float lx, float qx, float uu, float c, float z,
                                                const Args& a, double& px, bool flag_errors) {
  px = __builtin_nan("");
  bool acc = false;
  if (x >= 0 && x < a.V) {
    px = exp2(static_cast<double>(lx) * static_cast<double>(a.k2) - static_cast<double>(c)) /
         static_cast<double>(z);
    const double qd = qx;
    const double thr = px >= qd ? 1.0 : px / qd;  // no division when p >= q
    acc = static_cast<double>(uu) < thr;         // strict
    if (flag_errors && !(uu >= 0.f && uu < 1.f)) atomicOr(a.err, SV_DATA_UNIFORM);
  } else if (flag_errors && bad_id(a, x)) {
    atomicOr(a.err, SV_DATA_DRAFT_ID);
  }
  if (flag_errors && !(finite_pos(z) && finite_f(c))) atomicOr(a.err, SV_DATA_NONFINITE);
  return acc;
}
__device__ __forceinline__ bool accept_test(int x, float lx, float qx, float uu, float c, float z,
                                            const Args& a, double& px) {
  return accept_decision(x, lx, qx, uu, c, z, a, px, true);
}

// A pass-1 reference c as the fp64 draws take it. Pass 1 sums 2^(l k2 - c) with k2 the
// fp32 rounding of log2(e)/T, and the draws weigh entries by 2^(l k2d - c') with k2d =
// log2(e)/T itself, dividing by pass 1's z. With c' = c, the two sums differ by
// 2^(l (k2d - k2)) per term, an octave once |l k2| nears 2^24. With c' = c k2d / k2 (the
// same reference logit c / k2, scaled by k2d) they differ by 2^((l - c/k2)(k2d - k2)):
// within 3e-7 for every term within 30 octaves of the reference, at any |l k2|.
__device__ __forceinline__ double draw_ref(const Args& a, float c) { return static_cast<double>(c) * a.kr; }

// ============================================================== step 1
// Base-2 softmax state of entries [lo, hi) of one row: c = the scaled max (max(l) * k2,
// clamped to the fp32 range) and z = sum 2^(l k2 - c), kept per thread with a running max
// (thread tid of NT taking every NT-th group) and merged over the wave; every lane of the
// wave returns the wave's (c, z).
template <typename T, bool ALIGNED, int NT>
__device__ __forceinline__ void wave_row_lse(const T* row, int lo, int hi, float k2, int tid, float& c_out,
                                             float& z_out) {
  float m = -FLT_MAX, c = -FLT_MAX;  // running max of l and its scaled value
  float s[kGroup];
#pragma unroll
  for (int j = 0; j < kGroup; ++j) s[j] = 0.f;
  auto rebase = [&](float bm) {
    if (bm > m) {
      const float cn = fmaxf(bm * k2, -FLT_MAX);
      const float sc = fast_exp2(c - cn);
#pragma unroll
      for (int j = 0; j < kGroup; ++j) s[j] *= sc;
      m = bm;
      c = cn;
    }
  };
  if (ALIGNED) {
    const int g1 = hi >> 3;
    int g = (lo >> 3) + tid;
    for (; g + (kUnroll - 1) * NT < g1; g += kUnroll * NT) {
      float xv[kUnroll][kGroup];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) load_group(row, static_cast<size_t>(g + u * NT) * kGroup, xv[u]);
      float bm = xv[0][0];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int j = 0; j < kGroup; ++j) bm = fmaxf(bm, xv[u][j]);
      rebase(bm);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int j = 0; j < kGroup; ++j) s[j] += fast_exp2(fmaf(xv[u][j], k2, -c));
    }
    for (; g < g1; g += NT) {
      float xv[kGroup];
      load_group(row, static_cast<size_t>(g) * kGroup, xv);
      float bm = xv[0];
#pragma unroll
      for (int j = 1; j < kGroup; ++j) bm = fmaxf(bm, xv[j]);
      rebase(bm);
#pragma unroll
      for (int j = 0; j < kGroup; ++j) s[j] += fast_exp2(fmaf(xv[j], k2, -c));
    }
  } else {
    for (int e = lo + tid; e < hi; e += NT) {
      const float xv = load_one(row, e);
      rebase(xv);
      s[0] += fast_exp2(fmaf(xv, k2, -c));
    }
  }
  float z = ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float c2 = __shfl_xor(c, o), z2 = __shfl_xor(z, o);
    lse2_merge(c, z, c2, z2);
  }
  c_out = c;
  z_out = z;
}

// The same over an NT-thread block (kThreads by default): thread 0 returns the block's
// (C, Z); s_c, s_z are NT / 64-entry LDS scratch.
template <typename T, bool ALIGNED, int NT = kThreads>
__device__ __forceinline__ void block_row_lse(const T* row, int lo, int hi, float k2, float* s_c, float* s_z,
                                              float& C, float& Z) {
  float c, z;
  wave_row_lse<T, ALIGNED, NT>(row, lo, hi, k2, threadIdx.x, c, z);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    s_c[w] = c;
    s_z[w] = z;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    C = s_c[0];
    Z = s_z[0];
    for (int i = 1; i < NT / 64; ++i) lse2_merge(C, Z, s_c[i], s_z[i]);
  }
}

// Max raw logit of entries [lo, hi) of one row and its lowest index, over a kThreads
// block; thread 0 returns them. A range of -inf entries yields its first index. A NaN
// entry raises SV_DATA_NONFINITE in *err (the argmax is then unspecified).
template <typename T, bool ALIGNED>
__device__ __forceinline__ void block_row_argmax(const T* row, int lo, int hi, float* s_v, int* s_i, float& Vout,
                                                 int& Iout, int* err) {
  float bv = -INFINITY;
  float nw = -INFINITY;  // NaN watch
  int bi = INT_MAX;
  if (ALIGNED) {
    const int g1 = hi >> 3;
    int g = (lo >> 3) + threadIdx.x;
    if (g < g1) bi = g * kGroup;  // seed: a row of -inf still yields its first index
    for (; g + (kUnroll - 1) * kThreads < g1; g += kUnroll * kThreads) {
      float xv[kUnroll][kGroup];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) load_group(row, static_cast<size_t>(g + u * kThreads) * kGroup, xv[u]);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        nw = nan_watch(nw, xv[u]);
#pragma unroll
        for (int j = 0; j < kGroup; ++j)
          if (xv[u][j] > bv) {
            bv = xv[u][j];
            bi = (g + u * kThreads) * kGroup + j;
          }
      }
    }
    for (; g < g1; g += kThreads) {
      float xv[kGroup];
      load_group(row, static_cast<size_t>(g) * kGroup, xv);
      nw = nan_watch(nw, xv);
#pragma unroll
      for (int j = 0; j < kGroup; ++j)
        if (xv[j] > bv) {
          bv = xv[j];
          bi = g * kGroup + j;
        }
    }
  } else {
    int e = lo + threadIdx.x;
    if (e < hi) bi = e;
    for (; e < hi; e += kThreads) {
      const float xv = load_one(row, e);
      nw = nan_watch1(nw, xv);
      if (xv > bv) {
        bv = xv;
        bi = e;
      }
    }
  }
  flag_nan(nw, err, SV_DATA_NONFINITE);
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
    Vout = s_v[0];
    Iout = s_i[0];
    for (int i = 1; i < kWaves; ++i) argmax_merge(Vout, Iout, s_v[i], s_i[i]);
  }
}

template <typename T, bool ALIGNED, bool RAGGED, bool ACCEPT>
__global__ __launch_bounds__(kThreads) void k_rowstats(Args a) {
  __shared__ float s_c[kWaves], s_z[kWaves];
  const int d = blockIdx.x / a.split, k = blockIdx.x - d * a.split;
  const int b = RAGGED ? seq_of_row(a.cu, a.B, d) : d / a.gamma;
  const T* row = static_cast<const T*>(a.logits) + static_cast<size_t>(d + b) * a.V;
  // operands of the accept test, issued first so their latency hides under the stream;
  // a split row's operands are loaded by the split that holds the draft and kept for
  // the draw kernel, which then needs no dependent load to judge the row
  const int lo = k * a.span, hi = min(a.V, lo + a.span);
  int x = -1;
  float lx = 0.f, qx = 0.f, uu = 0.f;
  if (threadIdx.x == 0) {
    x = a.ids[d];
    if (ACCEPT) uu = a.u[d + b];
    if (ACCEPT ? (x >= 0 && x < a.V) : (x >= lo && x < hi)) {
      lx = load_one(row, x);
      qx = a.onehot ? 1.f : a.q[static_cast<size_t>(d) * a.V + x];
    }
  }
  float C, Z;
  block_row_lse<T, ALIGNED>(row, lo, hi, a.k2, s_c, s_z, C, Z);
  if (threadIdx.x == 0) {
    a.p1[blockIdx.x] = RowStat{C, Z};
    if (!ACCEPT && x >= lo && x < hi) a.lxq[d] = make_float2(lx, qx);
    if (ACCEPT) {
      double px;
      a.accept[d] = accept_test(x, lx, qx, uu, C, Z, a, px) ? 1 : 0;
      if (a.pdraft) a.pdraft[d] = static_cast<float>(px);
    }
  }
}

// Greedy twin: max raw logit of one split of one draft row and its lowest index; an
// unsplit row also records whether its draft equals that argmax.
template <typename T, bool ALIGNED, bool RAGGED, bool ACCEPT>
__global__ __launch_bounds__(kThreads) void k_rowargmax(Args a) {
  __shared__ float s_v[kWaves];
  __shared__ int s_i[kWaves];
  const int d = blockIdx.x / a.split, k = blockIdx.x - d * a.split;
  const int b = RAGGED ? seq_of_row(a.cu, a.B, d) : d / a.gamma;
  const T* row = static_cast<const T*>(a.logits) + static_cast<size_t>(d + b) * a.V;
  int x = -1;
  if (ACCEPT && threadIdx.x == 0) x = a.ids[d];
  const int lo = k * a.span, hi = min(a.V, lo + a.span);
  float V;
  int I;
  block_row_argmax<T, ALIGNED>(row, lo, hi, s_v, s_i, V, I, a.err);
  if (threadIdx.x == 0) {
    a.p1[blockIdx.x] = RowStat{V, __int_as_float(I)};
    if (ACCEPT) {
      // accept iff the draft equals the target argmax ([P1] ch.3 greedy; [P4])
      a.accept[d] = x == I ? 1 : 0;
      if (bad_id(a, x)) atomicOr(a.err, SV_DATA_DRAFT_ID);
    }
  }
}

// ============================================================== step 2: one workgroup per sequence
#ifndef SV_SEQ_WAVES
#define SV_SEQ_WAVES 16
#endif
#ifndef SV_RING
#define SV_RING 4
#endif
constexpr int kSeqWaves = SV_SEQ_WAVES;
constexpr int kSeqThreads = 64 * kSeqWaves;
constexpr int kIter = 64 * kGroup;          // entries a wave covers per sweep iteration (1 group per lane)
constexpr int kRing = SV_RING;              // sweep iterations held in registers (kRing - 1 in flight)
#ifndef SV_RING1
#define SV_RING1 4
#endif
constexpr int kRing1 = SV_RING1;            // the same for the one-launch row walk
#ifndef SV_NT_DRAW
#define SV_NT_DRAW 0
#endif
constexpr bool kNtDraw = SV_NT_DRAW;        // nontemporal loads for the table draw's sweep
constexpr int kPass = kSeqWaves * kIter;    // entries the block covers per re-sweep pass

// Raw bits of one group of 8 entries: one 16-byte vector for bf16, two for fp32.
template <typename T>
struct Raw {
  static constexpr int N = sizeof(T) / 2;
  uint4 v[N];
};

template <typename T> __device__ __forceinline__ uint32_t neg_inf_word();
template <> __device__ __forceinline__ uint32_t neg_inf_word<uint16_t>() { return 0xFF80FF80u; }
template <> __device__ __forceinline__ uint32_t neg_inf_word<float>() { return 0xFF800000u; }
__device__ __forceinline__ uint32_t elem_bits(const uint16_t* p, int e) { return p[e]; }
__device__ __forceinline__ uint32_t elem_bits(const float* p, int e) { return __float_as_uint(p[e]); }

// Group starting at entry e of `row`, known to lie inside the row (no check, so a
// loop of these keeps a fixed number of loads in flight).
template <typename T, bool NT = false>
__device__ __forceinline__ void load_raw_in(const T* __restrict__ row, int e, Raw<T>& r) {
  const uint4* p = reinterpret_cast<const uint4*>(row + e);
#pragma unroll
  for (int i = 0; i < Raw<T>::N; ++i) r.v[i] = load16<NT>(p + i);
}

// Group starting at entry e of `row`; entries at or past `lim` read as `fill`.
template <typename T, bool ALIGNED>
__device__ __forceinline__ void load_raw(const T* __restrict__ row, int e, int lim, Raw<T>& r, uint32_t fill) {
  if (ALIGNED) {
    if (e < lim) {
      const uint4* p = reinterpret_cast<const uint4*>(row + e);
#pragma unroll
      for (int i = 0; i < Raw<T>::N; ++i) r.v[i] = p[i];
    } else {
#pragma unroll
      for (int i = 0; i < Raw<T>::N; ++i) r.v[i] = make_uint4(fill, fill, fill, fill);
    }
  } else {
    uint32_t w[8];
    if (sizeof(T) == 2) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t lo = (e + 2 * k < lim) ? elem_bits(row, e + 2 * k) : (fill & 0xFFFFu);
        const uint32_t hi = (e + 2 * k + 1 < lim) ? elem_bits(row, e + 2 * k + 1) : (fill & 0xFFFFu);
        w[k] = lo | (hi << 16);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) w[k] = (e + k < lim) ? elem_bits(row, e + k) : fill;
    }
#pragma unroll
    for (int i = 0; i < Raw<T>::N; ++i) r.v[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
  }
}

__device__ __forceinline__ void unpack(const Raw<uint16_t>& r, float x[8]) {
  x[0] = bf16_lo(r.v[0].x); x[1] = bf16_hi(r.v[0].x); x[2] = bf16_lo(r.v[0].y); x[3] = bf16_hi(r.v[0].y);
  x[4] = bf16_lo(r.v[0].z); x[5] = bf16_hi(r.v[0].z); x[6] = bf16_lo(r.v[0].w); x[7] = bf16_hi(r.v[0].w);
}
__device__ __forceinline__ void unpack(const Raw<float>& r, float x[8]) {
  x[0] = __uint_as_float(r.v[0].x); x[1] = __uint_as_float(r.v[0].y);
  x[2] = __uint_as_float(r.v[0].z); x[3] = __uint_as_float(r.v[0].w);
  x[4] = __uint_as_float(r.v[1].x); x[5] = __uint_as_float(r.v[1].y);
  x[6] = __uint_as_float(r.v[1].z); x[7] = __uint_as_float(r.v[1].w);
}

// The per-sequence prologue shared by the sampling and greedy kernels: the first
// rejection n (g when every draft was accepted). Sampling also leaves each row's
// (c, z) in s_cz; greedy leaves each row's argmax in s_tok.
template <typename T, bool ACCEPT, bool GREEDY>
__device__ __forceinline__ int first_rejection(const Args& a, int b, int base, int g, float2* s_cz, int* s_tok,
                                               int* s_n) {
  if (threadIdx.x == 0) *s_n = g;
  __syncthreads();
  for (int i = threadIdx.x; i < g; i += kSeqThreads) {
    const int d = base + i;
    bool acc;
    if (ACCEPT) {
      const RowStat r = a.p1[d];
      if (GREEDY) s_tok[i] = __float_as_int(r.z);
      else s_cz[i] = make_float2(r.c, r.z);
      acc = a.accept[d] != 0;
    } else if (GREEDY) {
      float V = -INFINITY;
      int I = INT_MAX;
      for (int k = 0; k < a.split; ++k) {
        const RowStat r = a.p1[static_cast<size_t>(d) * a.split + k];
        argmax_merge(V, I, r.c, __float_as_int(r.z));
      }
      s_tok[i] = I;
      const int x = a.ids[d];
      acc = x == I;
      if (bad_id(a, x)) atomicOr(a.err, SV_DATA_DRAFT_ID);
    } else {
      float C = -FLT_MAX, Z = 0.f;
      for (int k = 0; k < a.split; ++k) {
        const RowStat r = a.p1[static_cast<size_t>(d) * a.split + k];
        lse2_merge(C, Z, r.c, r.z);
      }
      s_cz[i] = make_float2(C, Z);
      const int x = a.ids[d];
      const bool valid = x >= 0 && x < a.V;
      const float2 o = a.lxq[d];  // written by the split of step 1 that holds x (valid x only)
      const float lx = valid ? o.x : 0.f;
      const float qx = valid ? o.y : 0.f;
      double px;
      acc = accept_test(x, lx, qx, a.u[d + b], C, Z, a, px);
      if (a.pdraft) a.pdraft[d] = static_cast<float>(px);
    }
    if (!acc) atomicMin(s_n, i);
  }
  __syncthreads();
  return *s_n;
}

// Keeps the compiler from reordering memory operations across this point.
__device__ __forceinline__ void issue_order_fence() { asm volatile("" ::: "memory"); }

// Region geometry: wave w owns [w * rw, min(V, (w + 1) * rw)); rw is a multiple of
// kRing * kIter so that every region but the last holds whole rings of iterations.
__device__ __forceinline__ int region_width(int V) {
  const int per = (V + kSeqWaves - 1) / kSeqWaves;
  return (per + kRing * kIter - 1) / (kRing * kIter) * (kRing * kIter);
}

// Width of each of ns regions of a row for the split fp32 draw: ceil(V / ns) rounded up
// to whole sweep iterations, so short rows (V = 32000) still spread over every slice.
__host__ __device__ inline int iter_width(int V, int ns) {
  const int per = (V + ns - 1) / ns;
  return (per + kIter - 1) / kIter * kIter;
}

// One wave's fp64 sweep of entries [r0, r1) of a drawn row through a ring of kRing
// register buffers, e = 2^(l k2 - cr) by exp2_tab (KN = N k2, CN = N cr).
// Residual (qrow != null), with w = e - q Zq: s0 = sum max(w, 0), s1 = sum of q where
// w > 0, s2 = sum e. Bonus (qrow == null): s0 = the range's max logit (-inf when the
// range is empty), s1 = sum 2^((l - s0) k2), s2 = 0. The sums are wave-uniform.
template <typename T, bool ALIGNED>
__device__ __forceinline__ void draw_sweep(const T* lrow, const float* qrow, int r0, int r1, double KN, double CN,
                                           double Zq, const double* s_tab, double& s0, double& s1, double& s2) {
  const int lane = threadIdx.x & 63;
  // whole iterations are read without checks (only possible when aligned); the rest, masked
  const int nfull = ALIGNED ? (r1 - r0) / kIter : 0;
  const int mstart = r0 + nfull * kIter;
  const uint32_t linf = neg_inf_word<T>();
  if (qrow) {
    // residual max(0, p - q) ([P1] ch.3; [P3] 단계 3), normalisation deferred
    double D = 0.0, Zr = 0.0;
    float Q = 0.f;
    auto step = [&](const Raw<T>& lr, const Raw<float>& qr) {
      float x[kGroup], qv[kGroup];
      unpack(lr, x);
      unpack(qr, qv);
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        const double e = exp2_tab(fma(static_cast<double>(x[j]), KN, -CN), s_tab);
        const double w = fma(-static_cast<double>(qv[j]), Zq, e);
        D += fmax(w, 0.0);
        Q += w > 0.0 ? qv[j] : 0.f;
        Zr += e;
      }
    };
    if (nfull > 0) {
      Raw<T> Lb[kRing];
      Raw<float> Qb[kRing];
      const int eb = r0 + lane * kGroup, last = nfull - 1;
      auto at = [&](int it) { return eb + min(it, last) * kIter; };  // clamped: always in range
      // issue order pinned: the ring's wait counts assume the oldest buffer lands first
#pragma unroll
      for (int k = 0; k < kRing - 1; ++k) {
        load_raw_in(lrow, at(k), Lb[k]);
        load_raw_in(qrow, at(k), Qb[k]);
        issue_order_fence();
      }
      for (int it = 0; it < nfull; it += kRing) {
#pragma unroll
        for (int k = 0; k < kRing; ++k) {
          const int nb = (k + kRing - 1) % kRing;
          load_raw_in(lrow, at(it + k + kRing - 1), Lb[nb]);
          load_raw_in(qrow, at(it + k + kRing - 1), Qb[nb]);
          if (k == 0 || it + k < nfull) step(Lb[k], Qb[k]);
        }
      }
    }
    // the rest of the range, masked per lane (fills contribute nothing); the trip count
    // is the same for every lane of the wave
    for (int e0 = mstart; e0 < r1; e0 += kIter) {
      Raw<T> lr;
      Raw<float> qr;
      load_raw<T, ALIGNED>(lrow, e0 + lane * kGroup, r1, lr, linf);
      load_raw<float, ALIGNED>(qrow, e0 + lane * kGroup, r1, qr, 0u);
      step(lr, qr);
    }
    s0 = wave_sum(D);
    s1 = wave_sum(Q);
    s2 = wave_sum(Zr);
  } else {
    // bonus row ([P1] ch.2; [P3] 단계 3): running range max mw, sum 2^((l - mw) k2)
    float mw = -INFINITY;
    double mK = 0.0, sacc = 0.0;
    auto step = [&](const Raw<T>& lr) {
      float x[kGroup];
      unpack(lr, x);
      float bm = x[0];
#pragma unroll
      for (int j = 1; j < kGroup; ++j) bm = fmaxf(bm, x[j]);
      bm = wave_max_dpp(bm);
      if (bm > mw) {  // wave-uniform
        const double nK = static_cast<double>(bm) * KN;
        sacc *= mw > -INFINITY ? exp2_tab(mK - nK, s_tab) : 0.0;
        mw = bm;
        mK = nK;
      }
      if (mw > -INFINITY) {
#pragma unroll
        for (int j = 0; j < kGroup; ++j) sacc += exp2_tab(fma(static_cast<double>(x[j]), KN, -mK), s_tab);
      }
    };
    if (nfull > 0) {
      Raw<T> Lb[kRing];
      const int eb = r0 + lane * kGroup, last = nfull - 1;
      auto at = [&](int it) { return eb + min(it, last) * kIter; };
#pragma unroll
      for (int k = 0; k < kRing - 1; ++k) {
        load_raw_in(lrow, at(k), Lb[k]);
        issue_order_fence();
      }
      for (int it = 0; it < nfull; it += kRing) {
#pragma unroll
        for (int k = 0; k < kRing; ++k) {
          load_raw_in(lrow, at(it + k + kRing - 1), Lb[(k + kRing - 1) % kRing]);
          if (k == 0 || it + k < nfull) step(Lb[k]);
        }
      }
    }
    for (int e0 = mstart; e0 < r1; e0 += kIter) {  // wave-uniform trip count (step shuffles)
      Raw<T> lr;
      load_raw<T, ALIGNED>(lrow, e0 + lane * kGroup, r1, lr, linf);
      step(lr);
    }
    s0 = mw;
    s1 = wave_sum(sacc);
    s2 = 0.0;
  }
}

// What the search of a draw decided (wave-uniform; published through LDS).
struct DrawSel {
  double t;      // the target: u S (residual), u Z64 (from p) or u (Z64 - e(x_n))
  double P;      // the prefix before the selected region
  double Z64;    // sum of e over the row
  double delta;  // (Z64 - Zq) / Z64, residual only
  double S;      // residual mass (1 - p(x_n) for one-hot drafts; 0 for a bonus row)
  double ref;    // reference of e = 2^(l k2 - ref / N) in exp2_tab units
  int rs;        // selected region, -1 if no region has positive weight
  int kind;      // 0: residual; 1: degenerate residual (S <= 0), draw from p; 2: from p; 3: p without x_n
  int take_last; // no prefix crossed t (rounding, or u >= 1): the last positive entry
  int excl;      // the entry removed from p (kind 3), else -1
};

// Weight of a region (wave 0, one region per lane) from draw_sweep's sums (v0, v1, v2),
// given the row-wide values of the selection.
__device__ __forceinline__ double region_weight(int kind, double v0, double v1, double v2, double Z64,
                                                double delta, double ref, double KN, const double* s_tab) {
  if (kind == 0) return v0 / Z64 - v1 * delta;
  if (kind == 1) return v2;
  return v0 > -INFINITY ? v1 * exp2_tab(v0 * KN - ref, s_tab) : 0.0;
}

// The region where prefix + the inclusive scan of wgt first exceeds t (lanes < ns),
// else, or when `last` is set, the last region of positive weight; -1 if none. P
// returns the prefix before the selected region.
__device__ __forceinline__ int find_crossing(double wgt, bool live, double t, double prefix, bool last,
                                             double& P, int& take_last) {
  const double ex = wave_excl_scan(wgt);
  const unsigned long long cross = last ? 0ull : __ballot(live && prefix + ex + wgt > t);
  int rs = cross ? __ffsll(cross) - 1 : -1;
  P = prefix + __shfl(ex, rs < 0 ? 0 : rs);
  take_last = last ? 1 : 0;
  if (rs < 0) {
    take_last = 1;
    const unsigned long long pos = __ballot(live && wgt > 0.0);
    rs = pos ? 63 - __clzll(pos) : -1;
    P = rs < 0 ? prefix : prefix + __shfl(ex, rs);
  }
  return rs;
}

// The row-wide part of a draw's search (wave 0; lane r < ns holds region r's sums from
// draw_sweep): totals, residual mass, target and the region where the prefix crosses it.
// Raises the data flags of a non-finite normaliser or a uniform outside [0, 1).
__device__ __forceinline__ DrawSel draw_select(const Args& a, bool qres, bool oh, bool excl_ok, int xn, float lxn,
                                               int ns, int rw, double v0, double v1, double v2, double cr,
                                               double Zq, float uf, const double* s_tab) {
  const int lane = threadIdx.x & 63;
  const double KN = kExpScale * a.k2d;
  const double u = uf;
  const bool live = lane < ns;
  DrawSel d{};
  d.excl = -1;
  double wgt;
  if (qres) {
    d.Z64 = wave_sum(live ? v2 : 0.0);
    d.delta = (d.Z64 - Zq) / d.Z64;
    d.ref = kExpScale * cr;
    wgt = live ? region_weight(0, v0, v1, v2, d.Z64, d.delta, d.ref, KN, s_tab) : 0.0;
    d.S = wave_sum(wgt);
    d.kind = d.S > 0.0 ? 0 : 1;
    if (d.kind == 1) wgt = live ? v2 : 0.0;
    d.t = d.kind == 0 ? u * d.S : u * d.Z64;
  } else {
    double M = live ? v0 : -INFINITY;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmax(M, __shfl_xor(M, o));
    d.ref = M * KN;
    wgt = live ? region_weight(2, v0, v1, v2, 0.0, 0.0, d.ref, KN, s_tab) : 0.0;
    d.Z64 = wave_sum(wgt);
    d.kind = 2;
    d.t = u * d.Z64;
    if (oh) {
      // S = 1 - p(x_n); the region holding x_n loses e(x_n)
      const double ex_n = excl_ok ? exp2_tab(fma(static_cast<double>(lxn), KN, -d.ref), s_tab) : 0.0;
      d.S = (d.Z64 - ex_n) / d.Z64;
      if (d.S > 0.0) {
        d.kind = 3;
        d.excl = excl_ok ? xn : -1;
        if (excl_ok && live && lane == xn / rw) wgt = fmax(wgt - ex_n, 0.0);
        d.t = u * wave_sum(live ? wgt : 0.0);
      }
    }
  }
  d.rs = find_crossing(wgt, live, d.t, 0.0, false, d.P, d.take_last);
  if (lane == 0) {
    if (!(d.Z64 > 0.0 && d.Z64 <= DBL_MAX)) atomicOr(a.err, SV_DATA_NONFINITE);
    if (!(uf >= 0.f && uf < 1.f)) atomicOr(a.err, SV_DATA_UNIFORM);
  }
  return d;
}

// The block's re-sweep of entries [R0, R1) of a drawn row in passes of kPass entries
// (wave w scans the w-th kIter entries of a pass, lane l owns 8 consecutive entries):
// the first entry whose inclusive prefix (from sel.P) exceeds sel.t, else the last
// entry of positive weight; -1 if there is none. KN = N k2. Every thread of the block
// calls it and gets the result.
template <typename T, bool ALIGNED>
__device__ __forceinline__ int draw_resweep(const T* lrow, const float* qrow, int R0, int R1, const DrawSel& sel,
                                            double Zq, double KN, const double* s_tab) {
  __shared__ double s_wt[kSeqWaves];  // per-wave totals of a pass
  __shared__ int s_wc[kSeqWaves], s_wl[kSeqWaves];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t linf = neg_inf_word<T>();
  const int kind = sel.kind, excl = sel.excl;
  const bool take_last = sel.take_last != 0;
  const double t = sel.t, delta = sel.delta, ref = sel.ref;
  const double invZ = 1.0 / sel.Z64;
  double run = sel.P;
  int cand = INT_MAX, lastpos = -1;
  for (int p0 = R0; p0 < R1 && cand == INT_MAX; p0 += kPass) {
    const int e = p0 + wave * kIter + lane * kGroup;
    Raw<T> lr;
    float x[kGroup], qv[kGroup];
    load_raw<T, ALIGNED>(lrow, e, R1, lr, linf);
    unpack(lr, x);
    if (kind == 0) {
      Raw<float> qr;
      load_raw<float, ALIGNED>(qrow, e, R1, qr, 0u);
      unpack(qr, qv);
    }
    double rv[kGroup];
    double tot = 0.0;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const double ev = exp2_tab(fma(static_cast<double>(x[j]), KN, -ref), s_tab);
      double wv = ev;
      if (kind == 0) {
        const double w = fma(-static_cast<double>(qv[j]), Zq, ev);
        wv = w > 0.0 ? w * invZ - static_cast<double>(qv[j]) * delta : 0.0;
      }
      if (e + j == excl) wv = 0.0;
      rv[j] = wv;
      tot += wv;
    }
    const double lex = wave_excl_scan(tot);
    if (lane == 63) s_wt[wave] = lex + tot;
    __syncthreads();
    double acc = run;
    for (int w = 0; w < wave; ++w) acc += s_wt[w];
    acc += lex;
    int c2 = INT_MAX, lp = -1;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      acc += rv[j];
      if (!take_last && c2 == INT_MAX && acc > t) c2 = e + j;
      if (rv[j] > 0.0) lp = e + j;
    }
    c2 = wave_min_int(c2);
    lp = wave_max_int(lp);
    if (lane == 0) {
      s_wc[wave] = c2;
      s_wl[wave] = lp;
    }
    __syncthreads();
    int cm = INT_MAX, lm = -1;
    double tsum = run;
    for (int w = 0; w < kSeqWaves; ++w) {
      cm = min(cm, s_wc[w]);
      lm = max(lm, s_wl[w]);
      tsum += s_wt[w];
    }
    cand = cm;
    lastpos = max(lastpos, lm);
    run = tsum;
    __syncthreads();  // s_wt / s_wc / s_wl are rewritten by the next pass
  }
  return cand != INT_MAX ? cand : lastpos;
}

// The finish of the draw over ns <= 64 regions of width rw (region r covers
// [r rw, min(V, (r + 1) rw))): lane r < ns of wave 0 holds region r's sums (v0, v1, v2)
// from draw_sweep (the other lanes and waves are ignored). Wave 0 forms the totals and
// finds the region where the inclusive prefix first exceeds t; the block re-sweeps that
// region with an fp64 scan and writes emitted[n], the -1 padding after it and
// residual_sum[b]. uf is the sequence's uniform at position g (loaded by the caller
// before its sweep, off the draw's chain of dependent loads). Every thread of the block
// calls it.
template <typename T, bool ALIGNED>
__device__ __forceinline__ void draw_finish(const Args& a, int b, int base, int g, int n, double cr, double Zq,
                                            const double* s_tab, int xn, int ns, int rw, double v0, double v1,
                                            double v2, float uf) {
  __shared__ DrawSel s_sel;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int V = a.V;
  const bool residual = n < g;
  // one-hot drafts: max(0, p - onehot(x_n)) is p with x_n removed, drawn like a bonus row
  const bool oh = residual && a.onehot;
  const bool qres = residual && !oh;
  const T* lrow = static_cast<const T*>(a.logits) + static_cast<size_t>(base + b + (residual ? n : g)) * V;
  const float* qrow = qres ? a.q + static_cast<size_t>(base + n) * V : nullptr;
  if (wave == 0) {
    if (oh && xn < 0) xn = a.ids[base + n];
    const bool excl_ok = oh && xn >= 0 && xn < V;  // an invalid id removes nothing
    const float lxn = excl_ok ? load_one(lrow, xn) : 0.f;
    const DrawSel d = draw_select(a, qres, oh, excl_ok, xn, lxn, ns, rw, v0, v1, v2, cr, Zq, uf, s_tab);
    if ((threadIdx.x & 63) == 0) s_sel = d;
  }
  __syncthreads();
  const DrawSel sel = s_sel;
  int tok = V - 1;
  if (sel.rs >= 0) {
    const int R0 = min(V, sel.rs * rw), R1 = min(V, R0 + rw);
    const int r = draw_resweep<T, ALIGNED>(lrow, qrow, R0, R1, sel, Zq, kExpScale * a.k2d, s_tab);
    if (r >= 0) tok = r;
  }
  if (threadIdx.x == 0) {
    a.emitted[base + b + n] = tok;
    a.rsum[b] = residual ? static_cast<float>(sel.S) : 0.f;
  }
  for (int i = n + 1 + threadIdx.x; i <= g; i += kSeqThreads) a.emitted[base + b + i] = -1;
}

// The draw that ends a sequence's round ([P1] ch.2-3; [P2] "미리 그려놓고 한 번에 검증한다";
// [P3] 단계 3) in one workgroup: after a rejection at n < g, one token from
// norm(max(0, p_n - q_n)); when all g drafts were accepted, the bonus token from p_g.
// Writes emitted[n], the -1 padding after it and residual_sum[b]. For a residual, row
// n's statistics come in as a reference cref (in octaves) and Zq = sum 2^(l k2 - cref)
// over the row, exact or fp32-rounded (unused for the bonus). Wave w sweeps region w of
// the row; draw_finish does the rest. Every thread of the block calls it; s_tab holds
// the exp2_tab table.
template <typename T, bool ALIGNED>
__device__ __forceinline__ void final_draw(const Args& a, int b, int base, int g, int n, double cref,
                                           double Zq_in, const double* s_tab, int xn = -1) {
  __shared__ double s_reg[kSeqWaves][3];  // residual: (D, Q, Zr); bonus: (m, s, -)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int V = a.V;
  const bool residual = n < g;
  const bool qres = residual && !a.onehot;
  const T* lrow = static_cast<const T*>(a.logits) + static_cast<size_t>(base + b + (residual ? n : g)) * V;
  const float* qrow = qres ? a.q + static_cast<size_t>(base + n) * V : nullptr;
  const double cr = residual ? cref : 0.0;
  const double Zq = residual ? Zq_in : 0.0;
  const int rw = region_width(V);
  const int r0 = min(V, wave * rw), r1 = min(V, r0 + rw);
  const float uf = a.u[base + b + g];
  double s0, s1, s2;
  draw_sweep<T, ALIGNED>(lrow, qrow, r0, r1, kExpScale * a.k2d, kExpScale * cr, Zq, s_tab, s0, s1, s2);
  if (lane == 0) {
    s_reg[wave][0] = s0;
    s_reg[wave][1] = s1;
    s_reg[wave][2] = s2;
  }
  __syncthreads();
  const int r = lane < kSeqWaves ? lane : 0;
  draw_finish<T, ALIGNED>(a, b, base, g, n, cr, Zq, s_tab, xn, kSeqWaves, rw, s_reg[r][0], s_reg[r][1],
                          s_reg[r][2], uf);
}

// ============================================================== one-launch path
// One workgroup per sequence does the whole round. Pass 1 reads the draft rows in
// order and judges each as soon as its statistics are complete: the verification
// runs left to right and stops at the first rejection ([P2] "미리 그려놓고 한 번에
// 검증한다"; [P4] "이득의 크기는 두 숫자가 정한다"), so rows after it are not read
// (all rows are, when p(x) is requested for every draft). The 16 waves walk each row
// front to back in 512-entry chunks (wave w takes chunks w, w + 16, ...), through a
// register ring that runs on into the next row while a row is being judged. At a row
// end every wave merges the 16 partial (c, z) from LDS and runs the accept test itself
// (lane i holds row i's operands), so all waves reach the same decision without a
// second barrier. Pass 2 is final_draw.
constexpr int kFuseMaxGamma = 64;  // lane i judges row i

// One chunk of the row statistics: lanes whose group lies past the row (the partial
// last chunk; their load was clamped onto the row's last group) count with weight 0,
// which leaves the max unchanged too (that group is part of the row).
template <typename T>
__device__ __forceinline__ void stats_step(const Raw<T>& lr, float wgt, float k2, float& m, float& c,
                                           float (&sacc)[kGroup]) {
  float xv[kGroup];
  unpack(lr, xv);
  float bm = xv[0];
#pragma unroll
  for (int j = 1; j < kGroup; ++j) bm = fmaxf(bm, xv[j]);
  if (bm > m) {  // new running max: rebase the partial sums
    const float cn = fmaxf(bm * k2, -FLT_MAX);
    const float sc = fast_exp2(c - cn);
#pragma unroll
    for (int j = 0; j < kGroup; ++j) sacc[j] *= sc;
    m = bm;
    c = cn;
  }
#pragma unroll
  for (int j = 0; j < kGroup; ++j) sacc[j] = fmaf(wgt, fast_exp2(fmaf(xv[j], k2, -c)), sacc[j]);
}

// Walks the sequence's rows 0, 1, ... (row i at Lseq + i V) span by span: a span is
// kSeqWaves chunks of 512 entries, wave w reading chunk w of each span (so the block
// reads every row front to back). nitp, the spans per row rounded up to a multiple of
// kRing1, keeps every row starting at ring slot 0; the ring's loads run on into the next
// row while row_end(i) judges row i. A span's address is a scalar base plus the lane's
// fixed byte offset. With V >= one span (WIDE), the row's last span is read from
// V - kSpan, overlapping the one before, and lanes whose entry lies before
// (nsp - 1) kSpan must not count it (row_weight gives the lane's weight for the last
// span); otherwise the single span's lanes past V read the row's last group instead
// and must not count it. NT makes the loads nontemporal. Padding spans re-read the last span and are not handed to
// step. step(buf, k) gets the span index k < nsp; after_prologue() runs once the first
// loads are in flight; row_end(i) returns true to stop. row_ptr(i) gives walked row i
// (at most rows i and i + 1 are in flight: the ring is shorter than a row).
template <typename T, bool WIDE, bool NT, typename RowPtr, typename Pro, typename Step, typename RowEnd>
__device__ __forceinline__ void walk_rows_p(RowPtr&& row_ptr, int V, int g, Pro&& after_prologue, Step&& step,
                                            RowEnd&& row_end) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int kSpan = kSeqWaves * kIter;
  const int lane_off = wave * kIter + lane * kGroup;
  const uint32_t lane_byte = static_cast<uint32_t>(lane_off) * sizeof(T);
  const int nsp = (V + kSpan - 1) / kSpan;
  const int nitp = (nsp + kRing1 - 1) / kRing1 * kRing1;
  const int total = g * nitp;
  Raw<T> Lb[kRing1];
  int jl = 0, il = 0, kl = 0;  // next (flattened) iteration to load: row il, span kl
  auto issue = [&](Raw<T>& dst) {
    const T* rowp = row_ptr(il);
    if (WIDE) {
      const int e0 = kl < nsp - 1 ? kl * kSpan : V - kSpan;
      const char* sb = reinterpret_cast<const char*>(rowp + e0);
      const uint4* p = reinterpret_cast<const uint4*>(sb + lane_byte);
#pragma unroll
      for (int q = 0; q < Raw<T>::N; ++q) dst.v[q] = load16<NT>(p + q);
    } else {
      load_raw_in<T, NT>(rowp, min(lane_off, V - kGroup), dst);
    }
    if (jl < total - 1) {
      ++jl;
      if (++kl == nitp) {
        kl = 0;
        ++il;
      }
    }
  };
#pragma unroll
  for (int k = 0; k < kRing1 - 1; ++k) {
    issue(Lb[k]);
    issue_order_fence();
  }
  after_prologue();
  for (int i = 0; i < g; ++i) {
    for (int k0 = 0; k0 < nitp; k0 += kRing1) {
#pragma unroll
      for (int r = 0; r < kRing1; ++r) {
        issue(Lb[(r + kRing1 - 1) % kRing1]);
        const int k = k0 + r;
        if (k < nsp) step(Lb[r], k);
      }
    }
    if (row_end(i)) break;
  }
}
template <typename T, bool WIDE, bool NT, typename Pro, typename Step, typename RowEnd>
__device__ __forceinline__ void walk_rows(const T* Lseq, int V, int g, Pro&& after_prologue, Step&& step,
                                          RowEnd&& row_end) {
  walk_rows_p<T, WIDE, NT>([&](int i) { return Lseq + static_cast<size_t>(i) * V; }, V, g, after_prologue, step,
                           row_end);
}

// Weight of this lane's entries in the row's last span (see walk_rows).
template <bool WIDE>
__device__ __forceinline__ float last_span_weight(int V) {
  constexpr int kSpan = kSeqWaves * kIter;
  const int lane_off = (threadIdx.x >> 6) * kIter + (threadIdx.x & 63) * kGroup;
  const int nsp = (V + kSpan - 1) / kSpan;
  return (WIDE ? V - kSpan + lane_off >= (nsp - 1) * kSpan : lane_off < V) ? 1.f : 0.f;
}

// ---- bf16 value table: 2^(x k2) in fp64 for every bf16 x whose magnitude bits lie in
// [tlo, thi] (|x k2| < 990), both signs: entry 2 (mag - tlo) + sign. Magnitudes below tlo
// use the tlo entry (|x| below 2^-40 of the window top: relative error under 3e-12);
// above thi (and inf / NaN) they land on a sentinel pair of +inf after the window, so a
// sum over such a row is not finite and the exp2_tab path takes over.
constexpr int kTabBinades = 48;
constexpr int kTabEntries = 2 * kTabBinades * 128 + 2;

// clamp(x, 0, hi) in one instruction (hi >= 0)
__device__ __forceinline__ int med3_0(int x, int hi) {
  int r;
  asm("v_med3_i32 %0, %1, 0, %2" : "=v"(r) : "v"(x), "s"(hi));
  return r;
}
// tsent = thi + 1 - tlo, the sentinel's index
__device__ __forceinline__ double tab_lookup(uint32_t mag, uint32_t sgn, const double* sT, int tlo, int tsent) {
  return sT[2 * med3_0(static_cast<int>(mag) - tlo, tsent) + sgn];
}
// Fills sT. Within a binade the 128 values of x form an arithmetic sequence, so their
// 2^(x k2) form a geometric one: each of 768 pieces holds the 16 entries m = j, j + 8,
// ..., j + 120 of one (binade, sign), computes the first with exp2 and steps by
// R = 2^(8 dx k2) (relative error under 16 * 2^-52 + the exp2 error). Threads j = 0..7
// of the two signs of a binade write 16 adjacent entries per step, so the stores meet
// no LDS bank conflict. Workgroups of fewer than 770 threads take several pieces per
// thread. The caller syncs before the first lookup.
constexpr int kTabPiece = 16;
constexpr int kTabThreadsPerSign = 128 / kTabPiece;
static_assert(2 * kTabBinades * kTabThreadsPerSign + 2 <= 2 * kSeqThreads, "table pieces per thread");
__device__ __forceinline__ void tab_build(double* sT, const Args& a) {
  const int be_lo = a.tlo >> 7, nb = ((a.thi + 1) >> 7) - be_lo;
  for (int t = threadIdx.x; t < 2 * kTabBinades * kTabThreadsPerSign + 2; t += blockDim.x) {
    const int h = t / kTabThreadsPerSign, j = t % kTabThreadsPerSign;
    if (h < 2 * nb) {
      const int be = be_lo + (h >> 1);
      const double sgn = (h & 1) ? -1.0 : 1.0;
      // x = 2^(be - 127) (1 + m / 128) for be >= 1; subnormal binade: x = m 2^-133
      const double x0 = be >= 1 ? ldexp(1.0, be - 127) : 0.0;
      const double dx = ldexp(1.0, (be >= 1 ? be : 1) - 127 - 7);
      double v = exp2(sgn * (x0 + j * dx) * a.k2d);
      const double R = exp2(sgn * (kTabThreadsPerSign * dx) * a.k2d);
      double* dst = sT + 2 * (be * 128 + j - a.tlo) + (h & 1);
#pragma unroll
      for (int k = 0; k < kTabPiece; ++k) {
        dst[2 * kTabThreadsPerSign * k] = v;
        v *= R;
      }
    } else if (h == 2 * kTabBinades && j < 2) {  // two idle threads: the sentinel pair
      sT[2 * (a.thi + 1 - a.tlo) + j] = __builtin_inf();
    }
  }
}

// ---- the draw through the value table, in two parts: sweeps that form fp64 sums over
// sub-regions of the drawn row, and a finish that searches the sums and re-sweeps one
// sub-region. final_draw_tab runs both in one workgroup (16 sub-regions, one per wave);
// the split draw of the two-launch plan runs the sweeps of one row in several
// workgroups (k_draw_part), the last of which to finish also runs the finish.
constexpr int kMaxSlices = 4;                     // workgroups sweeping one row in the split draw
constexpr int kMaxSub = kMaxSlices * kSeqWaves;   // 64 sub-regions: lane k of a wave holds sub-region k
constexpr int kSplitMaxB = 1024;                  // sequences the split draw's workspace holds

// Width of one of ns sub-regions of a row: a multiple of kRing iterations, so a wave's
// sweep has no partial ring round except at the end of the row.
__host__ __device__ inline int sub_width(int V, int ns) {
  const int per = (V + ns - 1) / ns;
  return (per + kRing * kIter - 1) / (kRing * kIter) * (kRing * kIter);
}

// Byte offsets into the value table of the two bf16 values of one 32-bit word (low half
// first), both halves at once with packed 16-bit integer operations: the entry is
// 2 min(max(mag - tlo, 0), tsent) + sign, as in tab_lookup. tlo2 and tsent2 hold tlo and
// tsent in both halves; `three` is a register holding 3. (A packed operation takes an
// inline constant in its low half only, so op_sel_hi makes the high lane read the low
// half of the constants 15 and 2.)
__device__ __forceinline__ void tab_pair_offsets(uint32_t w, uint32_t tlo2, uint32_t tsent2, uint32_t three,
                                                 uint32_t& olo, uint32_t& ohi) {
  uint32_t m, i, s, e;
  asm("v_and_b32 %0, 0x7fff7fff, %1" : "=v"(m) : "v"(w));
  asm("v_pk_sub_u16 %0, %1, %2 clamp" : "=v"(i) : "v"(m), "s"(tlo2));  // saturates at 0
  asm("v_pk_min_u16 %0, %1, %2" : "=v"(i) : "v"(i), "s"(tsent2));
  asm("v_pk_lshrrev_b16 %0, 15, %1 op_sel_hi:[0,1]" : "=v"(s) : "v"(w));
  asm("v_pk_mad_u16 %0, %1, 2, %2 op_sel_hi:[1,0,1]" : "=v"(e) : "v"(i), "v"(s));
  asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_0"
      : "=v"(olo)
      : "v"(three), "v"(e));
  asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1"
      : "=v"(ohi)
      : "v"(three), "v"(e));
}

// The 8 table values of one group of raw bf16 words.
__device__ __forceinline__ void lookup8(const Raw<uint16_t>& lr, double (&e)[kGroup], const double* sT, int tlo,
                                        int tsent) {
  const uint32_t w[4] = {lr.v[0].x, lr.v[0].y, lr.v[0].z, lr.v[0].w};
  const uint32_t tlo2 = static_cast<uint32_t>(tlo) * 0x10001u, tsent2 = static_cast<uint32_t>(tsent) * 0x10001u;
  const uint32_t three = 3;
  const char* base = reinterpret_cast<const char*>(sT);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t olo, ohi;
    tab_pair_offsets(w[k], tlo2, tsent2, three, olo, ohi);
    e[2 * k] = *reinterpret_cast<const double*>(base + olo);
    e[2 * k + 1] = *reinterpret_cast<const double*>(base + ohi);
  }
}

// The drawn row of sequence b (row n after a rejection, the bonus row g otherwise) and,
// for a q residual, its q row.
__device__ __forceinline__ const uint16_t* drawn_row(const Args& a, int b, int base, int g, int n) {
  return static_cast<const uint16_t*>(a.logits) + static_cast<size_t>(base + b + (n < g ? n : g)) * a.V;
}
__device__ __forceinline__ const float* drawn_q(const Args& a, int base, int g, int n) {
  return n < g && !a.onehot ? a.q + static_cast<size_t>(base + n) * a.V : nullptr;
}

// One wave's sweep of entries [r0, r1) of a drawn row through the value table, through a
// ring of kRing register buffers. Residual (qrow != null): D = sum max(w, 0), Q = sum of
// q where w > 0, Zr = sum e, with w = e - q Zq; bonus: D = sum e. Totals in every lane.
__device__ __forceinline__ void tab_sweep(const uint16_t* lrow, const float* qrow, int r0, int r1, double Zq,
                                          const double* sT, int tlo, int tsent, double& Dout, double& Qout,
                                          double& Zout) {
  const int lane = threadIdx.x & 63;
  const int nfull = (r1 - r0) / kIter;
  const int mstart = r0 + nfull * kIter;
  if (qrow) {
    // residual max(0, p - q) ([P1] ch.3; [P3] 단계 3), normalisation deferred as in final_draw
    double D = 0.0, Zr = 0.0;
    float Q = 0.f;
    auto step = [&](const Raw<uint16_t>& lr, const Raw<float>& qr) {
      float qv[kGroup];
      unpack(qr, qv);
      double e[kGroup];
      lookup8(lr, e, sT, tlo, tsent);
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        const double w = fma(-static_cast<double>(qv[j]), Zq, e[j]);
        D += fmax(w, 0.0);
        Q += w > 0.0 ? qv[j] : 0.f;
        Zr += e[j];
      }
    };
    if (nfull > 0) {
      Raw<uint16_t> Lb[kRing];
      Raw<float> Qb[kRing];
      const int eb = r0 + lane * kGroup, last = nfull - 1;
      auto at = [&](int it) { return eb + min(it, last) * kIter; };
#pragma unroll
      for (int k = 0; k < kRing - 1; ++k) {
        load_raw_in<uint16_t, kNtDraw>(lrow, at(k), Lb[k]);
        load_raw_in<float, kNtDraw>(qrow, at(k), Qb[k]);
        issue_order_fence();
      }
      for (int it = 0; it < nfull; it += kRing) {
#pragma unroll
        for (int k = 0; k < kRing; ++k) {
          const int nb = (k + kRing - 1) % kRing;
          load_raw_in<uint16_t, kNtDraw>(lrow, at(it + k + kRing - 1), Lb[nb]);
          load_raw_in<float, kNtDraw>(qrow, at(it + k + kRing - 1), Qb[nb]);
          if (k == 0 || it + k < nfull) step(Lb[k], Qb[k]);
        }
      }
    }
    for (int e0 = mstart; e0 < r1; e0 += kIter) {  // the rest of the range; lanes past r1 idle
      Raw<uint16_t> lr;
      Raw<float> qr;
      const int e = e0 + lane * kGroup;
      load_raw_in<uint16_t, kNtDraw>(lrow, min(e, r1 - kGroup), lr);
      load_raw_in<float, kNtDraw>(qrow, min(e, r1 - kGroup), qr);
      if (e < r1) step(lr, qr);
    }
    Dout = wave_sum_dpp(D);
    Zout = wave_sum_dpp(Zr);
    Qout = wave_sum_dpp(static_cast<double>(Q));
  } else {
    // bonus row ([P1] ch.2; [P3] 단계 3): sum of 2^(l k2), no running max needed
    double sacc = 0.0;
    auto step = [&](const Raw<uint16_t>& lr) {
      double e[kGroup];
      lookup8(lr, e, sT, tlo, tsent);
      sacc += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    };
    if (nfull > 0) {
      Raw<uint16_t> Lb[kRing];
      const int eb = r0 + lane * kGroup, last = nfull - 1;
      auto at = [&](int it) { return eb + min(it, last) * kIter; };
#pragma unroll
      for (int k = 0; k < kRing - 1; ++k) {
        load_raw_in<uint16_t, kNtDraw>(lrow, at(k), Lb[k]);
        issue_order_fence();
      }
      for (int it = 0; it < nfull; it += kRing) {
#pragma unroll
        for (int k = 0; k < kRing; ++k) {
          load_raw_in<uint16_t, kNtDraw>(lrow, at(it + k + kRing - 1), Lb[(k + kRing - 1) % kRing]);
          if (k == 0 || it + k < nfull) step(Lb[k]);
        }
      }
    }
    for (int e0 = mstart; e0 < r1; e0 += kIter) {
      Raw<uint16_t> lr;
      const int e = e0 + lane * kGroup;
      load_raw_in<uint16_t, kNtDraw>(lrow, min(e, r1 - kGroup), lr);
      if (e < r1) step(lr);
    }
    Dout = wave_sum_dpp(sacc);
    Qout = 0.0;
    Zout = 0.0;
  }
}

// The finish of the table draw: lane k < ns of every wave holds sub-region k's sums
// (rD, rQ, rZ) (the same values in every wave, so all waves take the same decisions).
// Writes emitted[n], the -1 padding and residual_sum[b]. Returns false, having written
// nothing, when the drawn row holds a value outside the table (a sum is not finite).
// uf is the sequence's uniform at position g, loaded by the caller before its sweep.
__device__ __forceinline__ bool tab_finish(const Args& a, int b, int base, int g, int n, double Zq,
                                           const double* sT, int xn, int ns, double rD, double rQ, double rZ,
                                           float uf) {
  __shared__ double s_wt[2][kSeqWaves];  // re-sweep: per-wave totals, by pass parity
  __shared__ int s_cand, s_last;         // re-sweep: first crossing, last positive entry
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int V = a.V;
  const int tlo = a.tlo, tsent = a.thi + 1 - a.tlo;
  const int sw = sub_width(V, ns);
  const bool residual = n < g;
  // one-hot drafts: max(0, p - onehot(x_n)) is p with x_n removed, drawn like a bonus row
  const bool oh = residual && a.onehot;
  const bool qres = residual && !oh;
  const uint16_t* lrow = drawn_row(a, b, base, g, n);
  const float* qrow = drawn_q(a, base, g, n);
  if (oh && xn < 0) xn = a.ids[base + n];
  const bool excl_ok = oh && xn >= 0 && xn < V;  // an invalid id removes nothing
  const uint32_t lxn = excl_ok ? static_cast<uint32_t>(lrow[xn]) : 0u;
  if (threadIdx.x == 0) {
    s_cand = INT_MAX;
    s_last = -1;
  }

  // ---- totals and the sub-region where the inclusive prefix first exceeds t
  const double u = uf;
  const bool live = lane < ns;
  // a value outside the table reached the sentinel: the sub-region's sum is not finite
  if (__ballot(live && !((qres ? rZ : rD) <= DBL_MAX)) != 0) return false;
  int kind;  // 0: residual; 1: degenerate residual (S <= 0), draw from p; 2: from p; 3: p without x_n
  int excl = -1;
  double Z64, S = 0.0, delta = 0.0, t, wgt;
  if (qres) {
    Z64 = wave_sum_dpp(live ? rZ : 0.0);
    delta = (Z64 - Zq) / Z64;
    wgt = live ? rD / Z64 - rQ * delta : 0.0;
    S = wave_sum_dpp(wgt);
    kind = S > 0.0 ? 0 : 1;
    if (kind == 1) wgt = live ? rZ : 0.0;
    t = kind == 0 ? u * S : u * Z64;
  } else {
    wgt = live ? rD : 0.0;
    Z64 = wave_sum_dpp(wgt);
    kind = 2;
    t = u * Z64;
    if (oh) {
      // S = 1 - p(x_n); the sub-region holding x_n loses e(x_n)
      const double ex_n = excl_ok ? tab_lookup(lxn & 0x7FFFu, lxn >> 15, sT, tlo, tsent) : 0.0;
      S = (Z64 - ex_n) / Z64;
      if (S > 0.0) {
        kind = 3;
        excl = excl_ok ? xn : -1;
        if (excl_ok && live && lane == xn / sw) wgt = fmax(wgt - ex_n, 0.0);
        t = u * wave_sum_dpp(live ? wgt : 0.0);
      }
    }
  }
  const double inc = wave_incl_scan_dpp(wgt);
  const unsigned long long cross = __ballot(live && inc > t);
  int rs = cross ? __ffsll(cross) - 1 : -1;
  double run = readlane_d(inc - wgt, rs < 0 ? 0 : rs);
  bool take_last = false;
  if (rs < 0) {  // no crossing (rounding, or u >= 1): last positive-weight token
    take_last = true;
    const unsigned long long pos = __ballot(live && wgt > 0.0);
    rs = pos ? 63 - __clzll(pos) : -1;
    run = 0.0;
  }
  if (threadIdx.x == 0) {
    if (!(Z64 > 0.0 && Z64 <= DBL_MAX)) atomicOr(a.err, SV_DATA_NONFINITE);
    if (!(uf >= 0.f && uf < 1.f)) atomicOr(a.err, SV_DATA_UNIFORM);
  }

  // ---- re-sweep of sub-region r* in passes of kPass entries: wave w scans the w-th kIter
  // entries of a pass, lane l owns 8 consecutive entries; two barriers per pass
  int tok = V - 1;
  if (rs >= 0) {
    const int R0 = min(V, rs * sw), R1 = min(V, R0 + sw);
    const double invZ = 1.0 / Z64;
    int parity = 0;
    for (int p0 = R0; p0 < R1; p0 += kPass, parity ^= 1) {
      const int e = p0 + wave * kIter + lane * kGroup;
      const bool in = e < R1;
      Raw<uint16_t> lr;
      load_raw_in(lrow, min(e, R1 - kGroup), lr);
      float qv[kGroup];
      if (kind == 0) {
        Raw<float> qr;
        load_raw_in(qrow, min(e, R1 - kGroup), qr);
        unpack(qr, qv);
      }
      double ev[kGroup];
      lookup8(lr, ev, sT, tlo, tsent);
      double rv[kGroup];
      double tot = 0.0;
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        double wv = ev[j];
        if (kind == 0) {
          const double w = fma(-static_cast<double>(qv[j]), Zq, ev[j]);
          wv = w > 0.0 ? w * invZ - static_cast<double>(qv[j]) * delta : 0.0;
        }
        rv[j] = (in && e + j != excl) ? wv : 0.0;
        tot += rv[j];
      }
      const double linc = wave_incl_scan_dpp(tot);
      const double lex = linc - tot;
      if (lane == 63) s_wt[parity][wave] = linc;
      __syncthreads();
      double acc = run, tsum = run;
      for (int w2 = 0; w2 < kSeqWaves; ++w2) {
        const double v2 = s_wt[parity][w2];
        if (w2 < wave) acc += v2;
        tsum += v2;
      }
      acc += lex;
      int c2 = INT_MAX, lp = -1;
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        acc += rv[j];
        if (!take_last && c2 == INT_MAX && acc > t) c2 = e + j;
        if (rv[j] > 0.0) lp = e + j;
      }
      c2 = wave_min_int_dpp(c2);
      lp = wave_max_int_dpp(lp);
      if (lane == 0) {
        if (c2 != INT_MAX) atomicMin(&s_cand, c2);
        if (lp >= 0) atomicMax(&s_last, lp);
      }
      run = tsum;
      __syncthreads();
      if (s_cand != INT_MAX) break;
    }
    tok = s_cand != INT_MAX ? s_cand : (s_last >= 0 ? s_last : V - 1);
  }
  if (threadIdx.x == 0) {
    a.emitted[base + b + n] = tok;
    a.rsum[b] = residual ? static_cast<float>(S) : 0.f;
  }
  for (int i = n + 1 + threadIdx.x; i <= g; i += kSeqThreads) a.emitted[base + b + i] = -1;
  return true;
}


// The draw through the value table (bf16 rows) in one workgroup: the same arithmetic as
// final_draw with e = 2^(l k2) looked up instead of computed (reference 0); the residual's
// Zq comes in on that scale. Returns false, having written nothing, when the drawn row
// holds a value outside the table; the caller then runs final_draw.
__device__ __forceinline__ bool final_draw_tab(const Args& a, int b, int base, int g, int n, double Zq,
                                               const double* sT, int xn = -1) {
  __shared__ double s_reg[kSeqWaves][3];  // residual: (D, Q, Zr); bonus: (s, -, -)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sw = sub_width(a.V, kSeqWaves);
  const int r0 = min(a.V, wave * sw), r1 = min(a.V, r0 + sw);
  const float uf = a.u[base + b + g];
  double D, Q, Z;
  tab_sweep(drawn_row(a, b, base, g, n), drawn_q(a, base, g, n), r0, r1, Zq, sT, a.tlo, a.thi + 1 - a.tlo, D,
            Q, Z);
  if (lane == 0) {
    s_reg[wave][0] = D;
    s_reg[wave][1] = Q;
    s_reg[wave][2] = Z;
  }
  __syncthreads();
  const int k = lane < kSeqWaves ? lane : 0;
  return tab_finish(a, b, base, g, n, Zq, sT, xn, kSeqWaves, lane < kSeqWaves ? s_reg[k][0] : 0.0,
                    lane < kSeqWaves ? s_reg[k][1] : 0.0, lane < kSeqWaves ? s_reg[k][2] : 0.0, uf);
}
// Step 2 of the two-launch plan: one workgroup per sequence takes the row decisions of
// step 1, finds the first rejection and draws.
template <typename T, bool ALIGNED, bool RAGGED, bool ACCEPT>
__global__ __launch_bounds__(kSeqThreads) void k_sample_seq(Args a) {
  __shared__ double s_tab[kExpN];
  __shared__ float2 s_cz[kMaxGamma];
  __shared__ int s_n;
  const int b = blockIdx.x;
  int base, g;
  if (!seq_geom<RAGGED>(a, b, base, g)) {
    if (threadIdx.x == 0) {
      atomicOr(a.err, SV_DATA_CU_GAMMA);
      a.acc[b] = -1;
    }
    return;
  }
  exp_table_init(s_tab);
  if constexpr (ALIGNED && sizeof(T) == 2) {
    // bf16 rows: the draw through the value table, built while the decisions load
    __shared__ double sT[kTabEntries];
    const bool tab = a.tlo <= a.thi;
    if (tab) tab_build(sT, a);
    const int n = first_rejection<T, ACCEPT, false>(a, b, base, g, s_cz, nullptr, &s_n);
    for (int i = threadIdx.x; i < n; i += kSeqThreads) a.emitted[base + b + i] = a.ids[base + i];
    if (threadIdx.x == 0) a.acc[b] = n;
    __syncthreads();  // sT
    const double Zq = n < g ? static_cast<double>(s_cz[n].y) * exp2(draw_ref(a, s_cz[n].x)) : 0.0;
    if (tab && final_draw_tab(a, b, base, g, n, Zq, sT)) return;
    final_draw<T, ALIGNED>(a, b, base, g, n, n < g ? draw_ref(a, s_cz[n].x) : 0.0,
                           n < g ? static_cast<double>(s_cz[n].y) : 0.0, s_tab);
  } else {
    const int n = first_rejection<T, ACCEPT, false>(a, b, base, g, s_cz, nullptr, &s_n);
    for (int i = threadIdx.x; i < n; i += kSeqThreads) a.emitted[base + b + i] = a.ids[base + i];
    if (threadIdx.x == 0) a.acc[b] = n;
    final_draw<T, ALIGNED>(a, b, base, g, n, n < g ? draw_ref(a, s_cz[n].x) : 0.0,
                           n < g ? static_cast<double>(s_cz[n].y) : 0.0, s_tab);
  }
}

// The split draw of the two-launch plan (few sequences): workgroup (b, s) of k_draw_part
// finds sequence b's first rejection from step 1's decisions (every slice does it; only
// slice 0 writes the outputs of the scan), then sweeps slice s of the drawn row (16
// regions, one per wave) and stores the fp64 sums: bf16 rows through the value table,
// fp32 rows with exp2_tab as in final_draw. Each slice then counts itself done; the
// slice that completes the count (whichever finishes last) reads all 16 nslice sums and
// finishes the draw. No workgroup waits for another. The XCDs' L2 caches are not
// coherent with each other, so the sums and the count are written and read at system
// scope (past the L2s), and each wave waits for its sums' stores to complete before the
// count is taken; no cache-wide write-back or invalidate is needed.
template <typename T, bool RAGGED, bool ACCEPT>
__global__ __launch_bounds__(kSeqThreads) void k_draw_part(Args a) {
  constexpr bool kTab = sizeof(T) == 2;  // bf16 rows: the value table
  __shared__ double sT[kTab ? kTabEntries : 1];
  __shared__ double s_tab[kExpN];
  __shared__ float2 s_cz[kMaxGamma];
  __shared__ int s_n, s_last;
  const int b = blockIdx.x / a.nslice, s = blockIdx.x - b * a.nslice;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int base, g;
  if (!seq_geom<RAGGED>(a, b, base, g)) {
    if (s == 0 && threadIdx.x == 0) {
      atomicOr(a.err, SV_DATA_CU_GAMMA);
      a.acc[b] = -1;
    }
    return;
  }
  if constexpr (kTab)
    tab_build(sT, a);
  else
    exp_table_init(s_tab);
  const float uf = a.u[base + b + g];  // the draw's uniform, used by the finishing slice
  const int n = first_rejection<T, ACCEPT, false>(a, b, base, g, s_cz, nullptr, &s_n);
  if (s == 0) {
    for (int i = threadIdx.x; i < n; i += kSeqThreads) a.emitted[base + b + i] = a.ids[base + i];
    if (threadIdx.x == 0) a.acc[b] = n;
  }
  __syncthreads();  // sT / s_tab
  const double cr = n < g ? draw_ref(a, s_cz[n].x) : 0.0;
  const double zr = n < g ? static_cast<double>(s_cz[n].y) : 0.0;
  const int ns = kSeqWaves * a.nslice;
  const int sw = kTab ? sub_width(a.V, ns) : iter_width(a.V, ns);
  const int k = kSeqWaves * s + wave;
  const int r0 = min(a.V, k * sw), r1 = min(a.V, r0 + sw);
  double D, Q, Z;
  if constexpr (kTab) {
    tab_sweep(drawn_row(a, b, base, g, n), drawn_q(a, base, g, n), r0, r1, zr * exp2(cr), sT, a.tlo,
              a.thi + 1 - a.tlo, D, Q, Z);
  } else {
    const bool residual = n < g;
    const float* lrow = static_cast<const float*>(a.logits) + static_cast<size_t>(base + b + (residual ? n : g)) * a.V;
    draw_sweep<float, true>(lrow, drawn_q(a, base, g, n), r0, r1, kExpScale * a.k2d, kExpScale * cr, zr, s_tab, D,
                            Q, Z);
  }
  if (lane == 0) {
    double* dst = a.dsum + (static_cast<size_t>(b) * kMaxSub + k) * 3;
    __hip_atomic_store(dst, D, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(dst + 1, Q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(dst + 2, Z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the stores are complete before the count
  }
  __syncthreads();
  // the count is kept past the per-XCD L2 caches (system scope), where every slice sees it
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(&a.dcnt[b], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == a.nslice - 1;
  __syncthreads();
  if (!s_last) return;
  // the last slice: every slice's sums are complete in memory
  if (threadIdx.x == 0) __hip_atomic_store(&a.dcnt[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  double rD = 0.0, rQ = 0.0, rZ = 0.0;
  if (lane < ns) {  // every wave reads the same sums
    double* src = a.dsum + (static_cast<size_t>(b) * kMaxSub + lane) * 3;
    rD = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    rQ = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    rZ = __hip_atomic_load(src + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  if constexpr (kTab) {
    if (tab_finish(a, b, base, g, n, zr * exp2(cr), sT, -1, ns, rD, rQ, rZ, uf)) return;
    exp_table_init(s_tab);
    __syncthreads();  // s_tab
    final_draw<uint16_t, true>(a, b, base, g, n, cr, zr, s_tab);
  } else {
    draw_finish<float, true>(a, b, base, g, n, n < g ? cr : 0.0, n < g ? zr : 0.0, s_tab, -1, ns, sw, rD, rQ, rZ,
                             uf);
  }
}

// ============================================================== vocabulary-parallel verification
// One shard's part of a round when the vocabulary is cut into G contiguous column
// ranges, one per device: the rule ([P1] ch.3; [P3] 단계 3) is unchanged, only where
// the sums are taken moves. Shard k holds columns [vb[k], vb[k+1]) of every logits and
// q row. A round takes three steps per shard, with an all-gather of small records
// between them:
//   k_vs_rows:   per judged row, this shard's base-2 (c, z) over its columns (greedy: the
//                max and its lowest global index, bonus rows included) and, on the shard
//                that owns the draft id, l(x) and q(x): one 16-byte record per row;
//   k_vs_decide: merges the G records of each row in shard order, so every shard takes
//                the same decisions; writes the accepted count and tokens (greedy: every
//                output), then sweeps its columns of the drawn row in 16 regions: their
//                sums stay local, their total (24 bytes per sequence) is exchanged;
//   k_vs_finish: from the G totals, the shard whose columns hold the drawn token (the
//                last shard when no column has weight) searches its own regions,
//                re-sweeps one of them and writes the token, the -1 padding and S.
constexpr int kMaxShards = 64;
constexpr int kLocStride = 4 + 3 * kSeqWaves;  // per sequence: (cr, Zq, n, -), then each region's sums
struct ShardRec { float c, z, lx, qx; };
static_assert(sizeof(ShardRec) == 16 && kLocStride == 52, "record sizes stated in spec_verify.h");
struct VShard {
  int G, me, nrec;            // shards, this shard, records per shard
  int vb[kMaxShards + 1];     // column bounds of every shard
  ShardRec* rec;              // k_vs_rows: this shard's records [nrec]
  const ShardRec* all;        // k_vs_decide: every shard's records [G][nrec]
  double* part;               // k_vs_decide: this shard's totals [B][3]
  const double* part_all;     // k_vs_finish: every shard's totals [G][B][3]
  double* loc;                // this shard's per-sequence state [B][kLocStride]
};

// The shard whose columns hold id x, or -1 (x outside the vocabulary).
__device__ __forceinline__ int shard_of(const VShard& vs, int x) {
  int own = -1;
  for (int k = 0; k < vs.G; ++k)
    if (x >= vs.vb[k] && x < vs.vb[k + 1]) own = k;
  return own;
}

// Step 1: one kThreads workgroup per record. Records 0..R-1 are the draft rows; at T = 0
// records R..R+B-1 are the bonus rows. a.V is this shard's width.
template <typename T, bool ALIGNED, bool RAGGED, bool GREEDY>
__global__ __launch_bounds__(kThreads) void k_vs_rows(Args a, VShard vs) {
  __shared__ float s_c[kWaves], s_z[kWaves];
  __shared__ int s_i[kWaves];
  const int r = blockIdx.x;
  int b, t;
  if (r < a.R) {
    b = RAGGED ? seq_of_row(a.cu, a.B, r) : r / a.gamma;
    t = r + b;
  } else {  // the bonus row of sequence r - R
    b = r - a.R;
    const int c1 = RAGGED ? a.cu[b + 1] : (b + 1) * a.gamma;
    if (RAGGED && !(c1 >= 0 && c1 <= a.R)) {  // malformed offsets, flagged by k_vs_decide
      if (threadIdx.x == 0) vs.rec[r] = ShardRec{-INFINITY, __int_as_float(INT_MAX), 0.f, 0.f};
      return;
    }
    t = c1 + b;
  }
  const T* row = static_cast<const T*>(a.logits) + static_cast<size_t>(t) * a.V;
  const int v0 = vs.vb[vs.me];
  if constexpr (GREEDY) {
    float V;
    int I;
    block_row_argmax<T, ALIGNED>(row, 0, a.V, s_c, s_i, V, I, a.err);
    if (threadIdx.x == 0) vs.rec[r] = ShardRec{V, __int_as_float(I == INT_MAX ? INT_MAX : I + v0), 0.f, 0.f};
  } else {
    float lx = 0.f, qx = 0.f;
    if (threadIdx.x == 0) {  // the accept operands, issued before the stream
      const int x = a.ids[r];
      if (x >= v0 && x - v0 < a.V) {
        lx = load_one(row, x - v0);
        qx = a.q[static_cast<size_t>(r) * a.V + (x - v0)];
      }
    }
    float C, Z;
    block_row_lse<T, ALIGNED>(row, 0, a.V, a.k2, s_c, s_z, C, Z);
    if (threadIdx.x == 0) vs.rec[r] = ShardRec{C, Z, lx, qx};
  }
}

// Step 2: one workgroup per sequence. a.V is the whole vocabulary (ids are checked
// against it); the shard's width comes from vb.
template <typename T, bool ALIGNED, bool RAGGED, bool GREEDY>
__global__ __launch_bounds__(kSeqThreads) void k_vs_decide(Args a, VShard vs) {
  __shared__ double s_tab[kExpN];
  __shared__ float2 s_cz[kMaxGamma];
  __shared__ int s_tok[kMaxGamma + 1];
  __shared__ double s_reg[kSeqWaves][3];
  __shared__ int s_n;
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  double* loc = GREEDY ? nullptr : vs.loc + static_cast<size_t>(b) * kLocStride;
  int base, g;
  if (!seq_geom<RAGGED>(a, b, base, g)) {
    if (threadIdx.x == 0) {
      atomicOr(a.err, SV_DATA_CU_GAMMA);
      a.acc[b] = -1;
      if (!GREEDY) {
        loc[2] = -1.0;
        for (int j = 0; j < 3; ++j) vs.part[static_cast<size_t>(b) * 3 + j] = 0.0;
      }
    }
    return;
  }
  if (threadIdx.x == 0) s_n = g;
  if constexpr (GREEDY) {
    __syncthreads();
    for (int i = threadIdx.x; i <= g; i += kSeqThreads) {
      const int r = i < g ? base + i : a.R + b;
      float V = -INFINITY;
      int I = INT_MAX;
      for (int k = 0; k < vs.G; ++k) {
        const ShardRec e = vs.all[static_cast<size_t>(k) * vs.nrec + r];
        argmax_merge(V, I, e.c, __float_as_int(e.z));
      }
      s_tok[i] = I;
      if (i < g) {
        // accept iff the draft equals the target argmax ([P1] ch.3 greedy; [P4])
        const int x = a.ids[base + i];
        if (bad_id(a, x)) atomicOr(a.err, SV_DATA_DRAFT_ID);
        if (x != I) atomicMin(&s_n, i);
      }
    }
    __syncthreads();
    const int n = s_n;
    for (int i = threadIdx.x; i <= g; i += kSeqThreads)
      a.emitted[base + b + i] = i < n ? a.ids[base + i] : i == n ? s_tok[n] : -1;
    if (threadIdx.x == 0) {
      a.acc[b] = n;
      a.rsum[b] = 0.f;
    }
  } else {
    __syncthreads();  // s_n (the table is built after the accept tests, which do not use it)
    for (int i = threadIdx.x; i < g; i += kSeqThreads) {
      const int d = base + i;
      const int x = a.ids[d];
      const int own = shard_of(vs, x);
      float C = -FLT_MAX, Z = 0.f, lx = 0.f, qx = 0.f;
      for (int k = 0; k < vs.G; ++k) {
        const ShardRec e = vs.all[static_cast<size_t>(k) * vs.nrec + d];
        lse2_merge(C, Z, e.c, e.z);
        if (k == own) {
          lx = e.lx;
          qx = e.qx;
        }
      }
      s_cz[i] = make_float2(C, Z);
      double px;
      const bool acc = accept_test(x, lx, qx, a.u[d + b], C, Z, a, px);
      if (a.pdraft) a.pdraft[d] = static_cast<float>(px);
      if (!acc) atomicMin(&s_n, i);
    }
    exp_table_init(s_tab);
    __syncthreads();  // s_n, s_cz, s_tab
    const int n = s_n;
    for (int i = threadIdx.x; i < n; i += kSeqThreads) a.emitted[base + b + i] = a.ids[base + i];
    if (threadIdx.x == 0) a.acc[b] = n;
    // this shard's columns of the drawn row: the residual at row n, else the bonus row g
    const bool residual = n < g;
    const int Vs = vs.vb[vs.me + 1] - vs.vb[vs.me];
    const T* lrow = static_cast<const T*>(a.logits) + static_cast<size_t>(base + b + (residual ? n : g)) * Vs;
    const float* qrow = residual ? a.q + static_cast<size_t>(base + n) * Vs : nullptr;
    const double cr = residual ? draw_ref(a, s_cz[n].x) : 0.0;
    const double Zq = residual ? static_cast<double>(s_cz[n].y) : 0.0;
    const double KN = kExpScale * a.k2d;
    const int rw = iter_width(Vs, kSeqWaves);
    const int r0 = min(Vs, wave * rw), r1 = min(Vs, r0 + rw);
    double s0, s1, s2;
    draw_sweep<T, ALIGNED>(lrow, qrow, r0, r1, KN, kExpScale * cr, Zq, s_tab, s0, s1, s2);
    if (lane == 0) {
      s_reg[wave][0] = s0;
      s_reg[wave][1] = s1;
      s_reg[wave][2] = s2;
      loc[4 + 3 * wave] = s0;
      loc[5 + 3 * wave] = s1;
      loc[6 + 3 * wave] = s2;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      loc[0] = cr;
      loc[1] = Zq;
      loc[2] = n;
      double t0 = 0.0, t1 = 0.0, t2 = 0.0;
      if (residual) {  // (D, Q, Zr) add up
        for (int w = 0; w < kSeqWaves; ++w) {
          t0 += s_reg[w][0];
          t1 += s_reg[w][1];
          t2 += s_reg[w][2];
        }
      } else {  // (max, sum below it): rescale each region to the shard's max
        t0 = -INFINITY;
        for (int w = 0; w < kSeqWaves; ++w) t0 = fmax(t0, s_reg[w][0]);
        for (int w = 0; w < kSeqWaves; ++w)
          if (s_reg[w][0] > -INFINITY) t1 += s_reg[w][1] * exp2_tab(s_reg[w][0] * KN - t0 * KN, s_tab);
      }
      double* p = vs.part + static_cast<size_t>(b) * 3;
      p[0] = t0;
      p[1] = t1;
      p[2] = t2;
    }
  }
}

// Step 3: one workgroup per sequence; only the shard that owns the drawn token (or, with
// no weight anywhere, the last shard) writes emitted[n], the -1 padding and S.
template <typename T, bool ALIGNED, bool RAGGED>
__global__ __launch_bounds__(kSeqThreads) void k_vs_finish(Args a, VShard vs) {
  __shared__ double s_tab[kExpN];
  __shared__ DrawSel s_sel;
  __shared__ int s_own;
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int base, g;
  if (!seq_geom<RAGGED>(a, b, base, g)) return;  // flagged by k_vs_decide
  const double* loc = vs.loc + static_cast<size_t>(b) * kLocStride;
  // every operand of the selection, loaded at once ahead of the table: the shards'
  // totals (lane k: shard k), this shard's region sums (lane w: region w), cr, Zq, n, u
  double v0 = 0.0, v1 = 0.0, v2 = 0.0, g0 = 0.0, g1 = 0.0, g2 = 0.0;
  if (wave == 0) {
    if (lane < vs.G) {
      const double* p = vs.part_all + (static_cast<size_t>(lane) * a.B + b) * 3;
      v0 = p[0];
      v1 = p[1];
      v2 = p[2];
    }
    if (lane < kSeqWaves) {
      const double* lr = loc + 4 + 3 * lane;
      g0 = lr[0];
      g1 = lr[1];
      g2 = lr[2];
    }
  }
  const float uf = a.u[base + b + g];
  const double cr = loc[0], Zq = loc[1];
  const int n = static_cast<int>(loc[2]);
  exp_table_init(s_tab);
  __syncthreads();  // s_tab
  if (n < 0) return;
  const bool residual = n < g;
  const double KN = kExpScale * a.k2d;
  if (wave == 0) {
    // shards as regions: the one whose columns the prefix crosses t in
    DrawSel d = draw_select(a, residual, false, false, -1, 0.f, vs.G, 1, v0, v1, v2, cr, Zq, uf, s_tab);
    int own = d.rs < 0 ? (vs.me == vs.G - 1 ? 2 : 0) : d.rs == vs.me ? 1 : 0;
    if (own == 1) {  // this shard's regions, from the prefix before the shard
      const bool l2 = lane < kSeqWaves;
      const double w = l2 ? region_weight(d.kind, g0, g1, g2, d.Z64, d.delta, d.ref, KN, s_tab) : 0.0;
      double P;
      int tl;
      d.rs = find_crossing(w, l2, d.t, d.P, d.take_last != 0, P, tl);
      d.P = P;
      d.take_last = tl;
    }
    if (lane == 0) {
      s_sel = d;
      s_own = own;
    }
  }
  __syncthreads();
  if (s_own == 0) return;
  const DrawSel sel = s_sel;
  int tok = a.V - 1;
  if (s_own == 1 && sel.rs >= 0) {
    const int Vs = vs.vb[vs.me + 1] - vs.vb[vs.me];
    const int rw = iter_width(Vs, kSeqWaves);
    const T* lrow = static_cast<const T*>(a.logits) + static_cast<size_t>(base + b + (residual ? n : g)) * Vs;
    const float* qrow = residual ? a.q + static_cast<size_t>(base + n) * Vs : nullptr;
    const int R0 = min(Vs, sel.rs * rw), R1 = min(Vs, R0 + rw);
    const int r = draw_resweep<T, ALIGNED>(lrow, qrow, R0, R1, sel, Zq, KN, s_tab);
    if (r >= 0) tok = vs.vb[vs.me] + r;
  }
  if (threadIdx.x == 0) {
    a.emitted[base + b + n] = tok;
    a.rsum[b] = residual ? static_cast<float>(sel.S) : 0.f;
  }
  for (int i = n + 1 + threadIdx.x; i <= g; i += kSeqThreads) a.emitted[base + b + i] = -1;
}

// Pass 1: per row, z = sum 2^(l k2 - c) in fp32. Each wave keeps one reference c for its
// chunks of the row: the first chunk's max times k2, raised to a later chunk's max
// whenever an entry lies more than kRebaseOctaves above it (a wave-uniform branch: the
// sums are scaled by 2^(c_old - c_new)). Every term then has an exponent argument of at
// most kRebaseOctaves, whose rounding to fp32 is at most 2^-22 octave (1.7e-7 relative),
// and z stays below 2^21. At T = 1 the first chunk's reference holds for the whole row
// nearly always (8 octaves are 5.5 logits); low temperatures raise it a few times per
// row. A wave whose sum is not finite (infinite or NaN logits) redoes its chunks of the
// row with the running max, which raises the data flag. Returns n; s_cz[i] = (c, z) of
// each judged row.
template <typename T, bool WIDE, bool NT, typename Hook>
__device__ __forceinline__ int judge_rows_exact(const Args& a, int b, int base, int g, float2* s_cz, int* s_xn,
                                                Hook&& hook) {
  __shared__ float2 s_part[kSeqWaves];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int V = a.V;
  const T* Lseq = static_cast<const T*>(a.logits) + static_cast<size_t>(base + b) * V;
  const bool all_rows = a.pdraft != nullptr;
  const float k2 = a.k2;
  const int ir = min(lane, g - 1);
  const int x = a.ids[base + ir];
  const float uu = a.u[base + b + ir];
  const int xc = min(max(x, 0), V - 1);
  uint32_t lxb = 0;  // raw bits of l[x]
  float qx = 0.f;
  int n = g;
  constexpr int kSpan = kSeqWaves * kIter;
  const int lane_off = wave * kIter + lane * kGroup;
  const int nsp = (V + kSpan - 1) / kSpan;
  const float wlast = last_span_weight<WIDE>(V);
  float c = -FLT_MAX;  // this wave's reference for the current row
  float sacc[kGroup];
#pragma unroll
  for (int j = 0; j < kGroup; ++j) sacc[j] = 0.f;
  walk_rows<T, WIDE, NT>(
      Lseq, V, g,
      [&] {
        // the 32-bit word holding l[x] (rows are 16-byte aligned on this path)
        if constexpr (sizeof(T) == 2)
          lxb = reinterpret_cast<const uint32_t*>(Lseq + static_cast<size_t>(ir) * V)[xc >> 1];
        else
          lxb = elem_bits(Lseq + static_cast<size_t>(ir) * V, xc);
        qx = a.onehot ? 1.f : a.q[static_cast<size_t>(base + ir) * V + xc];
        hook();
      },
      [&](const Raw<T>& lr, int k) {
        float t[kGroup];  // exponent arguments l k2 - c
        {
          float xv[kGroup];
          unpack(lr, xv);
#pragma unroll
          for (int j = 0; j < kGroup; ++j) t[j] = fmaf(xv[j], k2, -c);
        }
        float tm = t[0];
#pragma unroll
        for (int j = 1; j < kGroup; ++j) tm = fmaxf(tm, t[j]);
        // a new reference when an entry of the chunk lies more than kRebaseOctaves above
        // the current one (at the row's first chunk c is -FLT_MAX: always)
        if (__builtin_expect(__ballot(tm > kRebaseOctaves) != 0, 0)) {
          float xv[kGroup];
          unpack(lr, xv);
          float bm = xv[0];
#pragma unroll
          for (int j = 1; j < kGroup; ++j) bm = fmaxf(bm, xv[j]);
          const float cn = fmaxf(wave_max_dpp(bm) * k2, -FLT_MAX);
          const float sc = fast_exp2(c - cn);
#pragma unroll
          for (int j = 0; j < kGroup; ++j) {
            sacc[j] *= sc;
            t[j] = fmaf(xv[j], k2, -cn);
          }
          c = cn;
        }
        const float wgt = k == nsp - 1 ? wlast : 1.f;
#pragma unroll
        for (int j = 0; j < kGroup; ++j) sacc[j] = fmaf(wgt, fast_exp2(t[j]), sacc[j]);
      },
      [&](int i) {
        float z = wave_sum(((sacc[0] + sacc[1]) + (sacc[2] + sacc[3])) + ((sacc[4] + sacc[5]) + (sacc[6] + sacc[7])));
        float cw = c;
        if (!(z <= FLT_MAX)) {  // not finite (data errors): this wave's chunks again, running max
          const T* rowp = Lseq + static_cast<size_t>(i) * V;
          float m = -FLT_MAX;
          cw = -FLT_MAX;
#pragma unroll
          for (int j = 0; j < kGroup; ++j) sacc[j] = 0.f;
          for (int k = 0; k < nsp; ++k) {
            Raw<T> lr;
            const int e = WIDE ? (k < nsp - 1 ? k * kSpan : V - kSpan) + lane_off : min(lane_off, V - kGroup);
            load_raw_in(rowp, e, lr);
            stats_step<T>(lr, k == nsp - 1 ? wlast : 1.f, k2, m, cw, sacc);
          }
          z = ((sacc[0] + sacc[1]) + (sacc[2] + sacc[3])) + ((sacc[4] + sacc[5]) + (sacc[6] + sacc[7]));
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) {
            const float c2 = __shfl_xor(cw, o), z2 = __shfl_xor(z, o);
            lse2_merge(cw, z, c2, z2);
          }
        }
        if (lane == 0) s_part[wave] = make_float2(cw, z);
        c = -FLT_MAX;
#pragma unroll
        for (int j = 0; j < kGroup; ++j) sacc[j] = 0.f;
        __syncthreads();
        // every wave merges the partials in the same order and takes the same decision
        static_assert(kSeqWaves == 16, "one DPP row holds the wave partials");
        const float2 pz = s_part[lane & (kSeqWaves - 1)];
        float C, Z;
        merge_row16(pz.x, pz.y, C, Z);
        // lx, qx were loaded behind the ring's first loads: keep their uses here, inside
        // the row loop, so that waiting for them never drains the ring
        asm volatile("" : "+v"(lxb), "+v"(qx));
        const float lx = sizeof(T) == 2 ? bf16_word_half(lxb, xc & 1) : __uint_as_float(lxb);
        bool acc = true;
        double px = 0.0;
        if (lane == i) acc = accept_decision(x, lx, qx, uu, C, Z, a, px, wave == 0);
        if (wave == 0 && lane == i) {
          if (a.pdraft) a.pdraft[base + i] = static_cast<float>(px);
          s_cz[i] = make_float2(C, Z);
        }
        const bool rej = __ballot(!acc) != 0;
        __syncthreads();  // s_part is rewritten by the next row
        if (rej && n == g) {
          n = i;
          if (!all_rows) return true;  // with p(x) wanted, the remaining rows are still judged
        }
        return false;
      });
  // the accepted drafts and the count, from the operands already in wave 0's lanes
  if (wave == 0) {
    if (lane < n) a.emitted[base + b + lane] = x;
    if (lane == 0) a.acc[b] = n;
    if (lane == n) *s_xn = x;  // the rejected draft (n < g)
  }
  return n;
}

// The order in which the one-launch plan takes the sequences of a ragged batch with
// more sequences than compute units: longest draft first, a counting sort by gamma_b,
// descending (the order of equal gamma_b is arbitrary). Workgroups are dispatched in
// index order as compute units free up, so the short sequences go last and the step
// ends with less imbalance. A malformed gamma_b lands in some bin, so every sequence
// appears once; the verification kernel flags it. One workgroup.
constexpr int kOrderThreads = 1024;
constexpr int kOrderKeep = 8;  // bins a thread keeps in registers between the two passes
__global__ __launch_bounds__(kOrderThreads) void k_order_by_gamma(Args a) {
  __shared__ int s_bin[kFuseMaxGamma + 1];
  auto bin = [&](int b) {
    const int g = static_cast<int>(static_cast<uint32_t>(a.cu[b + 1]) - static_cast<uint32_t>(a.cu[b]));
    return kFuseMaxGamma - min(max(g, 0), kFuseMaxGamma);
  };
  for (int i = threadIdx.x; i <= kFuseMaxGamma; i += kOrderThreads) s_bin[i] = 0;
  __syncthreads();
  int keep[kOrderKeep];
#pragma unroll
  for (int k = 0; k < kOrderKeep; ++k) {
    const int b = threadIdx.x + k * kOrderThreads;
    keep[k] = b < a.B ? bin(b) : 0;
  }
#pragma unroll
  for (int k = 0; k < kOrderKeep; ++k)
    if (threadIdx.x + k * kOrderThreads < a.B) atomicAdd(&s_bin[keep[k]], 1);
  for (int b = threadIdx.x + kOrderKeep * kOrderThreads; b < a.B; b += kOrderThreads) atomicAdd(&s_bin[bin(b)], 1);
  __syncthreads();
  if (threadIdx.x == 0) {  // exclusive prefix over the bins
    int run = 0;
    for (int i = 0; i <= kFuseMaxGamma; ++i) {
      const int c = s_bin[i];
      s_bin[i] = run;
      run += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kOrderKeep; ++k) {
    const int b = threadIdx.x + k * kOrderThreads;
    if (b < a.B) a.order[atomicAdd(&s_bin[keep[k]], 1)] = b;
  }
  for (int b = threadIdx.x + kOrderKeep * kOrderThreads; b < a.B; b += kOrderThreads)
    a.order[atomicAdd(&s_bin[bin(b)], 1)] = b;
}

// ============================================================== small batches, one launch
// With fewer sequences than compute units one launch of B x gamma x split workgroups
// reads every draft row in parallel. Workgroup w = b * W + j (W = gamma * split per
// sequence, j = i * split + k) takes chunk k of draft row i of sequence b: it computes the
// chunk's base-2 softmax state (the chunk holding the draft also the draft's logit and q
// entry) and stores it as a record of four 64-bit words, the value in the high half and
// the call's tag in the low half. Wave 0 of every workgroup of the sequence then waits
// until the sequence's W records carry the tag, merges each row's records in chunk order
// and runs the fp64 accept tests of all rows ([P1] ch.3; [P3] 단계 3); every workgroup
// of the sequence reaches the same first rejection n (same records, same order). The
// drawn row (the residual of row n, or the bonus row when every draft is accepted; [P1]
// ch.2) is cut into up to 64 units, unit u swept by wave u of the sequence's workgroups,
// so the whole group sweeps it at once; each wave stores its unit's fp64 sums as six
// tagged words (each 32-bit half of a sum beside the tag). The wave of unit 0 then waits
// until every unit's words carry the tag and finishes the draw: the search over the unit
// sums, the re-sweep of the selected unit, the sequence's outputs. With gamma = 0 a
// sequence has one workgroup, which draws from its bonus row directly.
//
// Hand-offs between workgroups: the words handed over are stored and loaded with relaxed
// atomics at system scope, which gfx950 executes as global stores and loads with sc0 sc1:
// they bypass the per-XCD L2 caches (not coherent with each other) and are performed at
// memory, each 64-bit word at once. A reader takes a value only from a word that carries
// this call's tag, and every word of a value carries it, so it never mixes words of two
// calls and needs no other signal; no word is reset between calls (an older call's words
// carry an older tag; the tag is a 32-bit count of the context's launches of this plan).
// Every wait is bounded; one that runs out raises SV_DATA_STALL (that call's outputs are
// then not valid). The host sizes the grid so that every workgroup is resident at once,
// and a wait then lasts only until the other workgroups of the group have stored their
// part. With fewer resident (other work on the device) the groups still finish: a group's
// workgroups are contiguous in dispatch order, so the earliest unfinished group has all
// of its workgroups dispatched, and it never waits on a later one.
#ifndef SV_GRP_THREADS
#define SV_GRP_THREADS 256
#endif
constexpr int kGrpThreads = SV_GRP_THREADS;
constexpr int kGrpWaves = kGrpThreads / 64;
constexpr int kGrpMaxW = 64;            // workgroups of one sequence (records of one lane each)
constexpr int kGrpMaxUnits = 64;        // units of a drawn row (unit sums of one lane each)
constexpr int kGrpMaxItems = 2048;      // workgroups of one launch (records in the workspace)
constexpr int kGrpSpinCap = 1 << 20;    // polls of a wait before it gives up (SV_DATA_STALL)
constexpr int kSumWords = 6;            // words of a unit's three fp64 sums, each half tagged

__device__ __forceinline__ void store_sys(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ unsigned long long load_sys(const unsigned long long* p) {
  return __hip_atomic_load(const_cast<unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ unsigned long long rec_word(float v, unsigned tag) {
  return (static_cast<unsigned long long>(__float_as_uint(v)) << 32) | tag;
}
__device__ __forceinline__ float rec_value(unsigned long long w) { return __uint_as_float(static_cast<uint32_t>(w >> 32)); }
__device__ __forceinline__ bool rec_tagged(unsigned long long w, unsigned tag) { return static_cast<uint32_t>(w) == tag; }

// A sequence's draw: pass-1 statistics of the drawn row (z, c; 0 for a bonus draw), n, g,
// the row base, the rejected draft (the excluded token of one-hot drafts), the sequence,
// the uniform.
struct GroupDraw {
  double zr, cr;
  int n, g, base, xn, b;
  float uf;
};

__device__ __forceinline__ double uniform_d(double v) {
  return __hiloint2double(__builtin_amdgcn_readfirstlane(__double2hiint(v)),
                          __builtin_amdgcn_readfirstlane(__double2loint(v)));
}
// The same values, held in scalar registers (they are the same in every lane).
__device__ __forceinline__ GroupDraw uniform_draw(const GroupDraw& d) {
  GroupDraw u;
  u.zr = uniform_d(d.zr);
  u.cr = uniform_d(d.cr);
  u.n = __builtin_amdgcn_readfirstlane(d.n);
  u.g = __builtin_amdgcn_readfirstlane(d.g);
  u.base = __builtin_amdgcn_readfirstlane(d.base);
  u.xn = __builtin_amdgcn_readfirstlane(d.xn);
  u.b = __builtin_amdgcn_readfirstlane(d.b);
  u.uf = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(d.uf)));
  return u;
}

// The drawn row of d and, for a residual draw with drafts of real probabilities, the
// draft row's q.
template <typename T>
__device__ __forceinline__ const T* drawn_row(const Args& a, const GroupDraw& d) {
  return static_cast<const T*>(a.logits) + static_cast<size_t>(d.base + d.b + d.n) * a.V;
}
__device__ __forceinline__ const float* drawn_q(const Args& a, const GroupDraw& d) {
  return d.n < d.g && !a.onehot ? a.q + static_cast<size_t>(d.base + d.n) * a.V : nullptr;
}

// One wave's re-sweep of entries [R0, R1) of a drawn row (R0 and R1 multiples of kGroup)
// through a ring of four iterations (three for fp32 logits): the first entry whose inclusive prefix (from sel.P)
// exceeds sel.t, else the last entry of positive weight, -1 if none. e = 2^(l k2 - ref)
// by exp2_tab, weighted as draw_select's kind says.
template <typename T>
__device__ __forceinline__ int wave_resweep(const T* lrow, const float* qrow, int R0, int R1, const DrawSel& sel,
                                            double Zq, double KN, const double* s_tab) {
  const int lane = threadIdx.x & 63;
  const int kind = sel.kind, excl = sel.excl;
  const bool take_last = sel.take_last != 0;
  const double t = sel.t, delta = sel.delta, ref = sel.ref;
  const double invZ = 1.0 / sel.Z64;
  const int nit = (R1 - R0 + kIter - 1) / kIter;
  double run = sel.P;
  int lastpos = -1;
  constexpr int kR = sizeof(T) == 2 ? 4 : 3;  // iterations held in registers (all but one in flight)
  Raw<T> Lb[kR];
  Raw<float> Qb[kR];
  auto issue = [&](int it, int slot) {
    const int e = min(R0 + min(it, nit - 1) * kIter + lane * kGroup, R1 - kGroup);
    load_raw_in(lrow, e, Lb[slot]);
    if (kind == 0) load_raw_in(qrow, e, Qb[slot]);
  };
#pragma unroll
  for (int k = 0; k < kR - 1; ++k) {
    issue(k, k);
    issue_order_fence();
  }
  for (int it0 = 0; it0 < nit; it0 += kR) {
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int it = it0 + r;
      issue(it + kR - 1, (r + kR - 1) % kR);
      if (it >= nit) continue;
      const int e = R0 + it * kIter + lane * kGroup;
      const bool in = e < R1;
      float x[kGroup];
      unpack(Lb[r], x);
      float qv[kGroup];
      if (kind == 0) unpack(Qb[r], qv);
      double rv[kGroup];
      double tot = 0.0;
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        const double ev = exp2_tab(fma(static_cast<double>(x[j]), KN, -ref), s_tab);
        double wv = ev;
        if (kind == 0) {
          const double w = fma(-static_cast<double>(qv[j]), Zq, ev);
          wv = w > 0.0 ? w * invZ - static_cast<double>(qv[j]) * delta : 0.0;
        }
        rv[j] = (in && e + j != excl) ? wv : 0.0;
        tot += rv[j];
      }
      const double inc = wave_incl_scan_dpp(tot);
      double acc = run + (inc - tot);
      int c2 = INT_MAX, lp = -1;
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        acc += rv[j];
        if (!take_last && c2 == INT_MAX && acc > t) c2 = e + j;
        if (rv[j] > 0.0) lp = e + j;
      }
      c2 = wave_min_int_dpp(c2);
      lp = wave_max_int_dpp(lp);
      run += readlane_d(inc, 63);
      lastpos = max(lastpos, lp);
      if (c2 != INT_MAX) return c2;
    }
  }
  return lastpos;
}

// The finish of a sequence's draw by one wave, unit u's sums in lane u: the search, the
// re-sweep of the selected unit, and the sequence's outputs (accepted count, the accepted
// drafts, the drawn token, the -1 padding, residual_sum). Lane i holds draft i's id
// (gamma <= 64).
template <typename T>
__device__ __forceinline__ void group_finish(const Args& a, const GroupDraw& d, double v0, double v1, double v2,
                                             const double* s_tab, int myid) {
  const int lane = threadIdx.x & 63;
  const int V = a.V;
  const bool residual = d.n < d.g;
  const bool oh = residual && a.onehot;
  const bool qres = residual && !oh;
  const T* lrow = drawn_row<T>(a, d);
  const float* qrow = drawn_q(a, d);
  const bool excl_ok = oh && d.xn >= 0 && d.xn < V;  // an invalid id removes nothing
  const float lxn = excl_ok ? load_one(lrow, d.xn) : 0.f;
  const DrawSel sel = draw_select(a, qres, oh, excl_ok, d.xn, lxn, a.nunits, a.uw, v0, v1, v2,
                                  residual ? d.cr : 0.0, residual ? d.zr : 0.0, d.uf, s_tab);
  int tok = -1;
  if (sel.rs >= 0) {
    const int R0 = min(V, sel.rs * a.uw), R1 = min(V, R0 + a.uw);
    tok = wave_resweep<T>(lrow, qrow, R0, R1, sel, residual ? d.zr : 0.0, kExpScale * a.k2d, s_tab);
  }
  if (tok < 0) tok = V - 1;
  const int out = d.base + d.b;
  if (lane < d.n) a.emitted[out + lane] = myid;
  for (int i = d.n + 1 + lane; i <= d.g; i += 64) a.emitted[out + i] = -1;
  if (lane == 0) {
    a.emitted[out + d.n] = tok;
    a.acc[d.b] = d.n;
    a.rsum[d.b] = residual ? static_cast<float>(sel.S) : 0.f;
  }
}

template <typename T>
__global__ __launch_bounds__(kGrpThreads, 4) void k_verify_group(Args a) {
  __shared__ double s_tab[kExpN];
  __shared__ float s_c[kGrpWaves], s_z[kGrpWaves];
  __shared__ GroupDraw s_d;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int V = a.V, g = a.gamma, S = a.split;
  const int W = g > 0 ? g * S : 1;  // workgroups of a sequence
  const int b = static_cast<int>(blockIdx.x) / W, j = static_cast<int>(blockIdx.x) - b * W;
  const int base = b * g;
  exp_table_init(s_tab);
  int xv = 0;  // wave 0, lane i: draft i's id
  if (g > 0) {
    const int i = j / S, k = j - i * S;  // chunk k of draft row i
    const int d = base + i;
    const T* row = static_cast<const T*>(a.logits) + static_cast<size_t>(d + b) * V;
    const int lo = k * a.span, hi = min(V, lo + a.span);
    // wave 0: the sequence's drafts and uniforms (lane i: row i), loaded ahead of pass 1
    const int ii = min(lane, g - 1);
    float uu = 0.f, uf = 0.f;
    float lx = 0.f, qx = 0.f;
    if (wave == 0) {
      xv = a.ids[base + ii];
      uu = a.u[base + ii + b];
      uf = a.u[base + b + g];
      if (lane == 0) {  // the accept operands of this chunk
        const int x = a.ids[d];
        if (x >= lo && x < hi) {
          lx = load_one(row, x);
          qx = a.onehot ? 1.f : a.q[static_cast<size_t>(d) * V + x];
        }
      }
    }
    float C, Z;
    block_row_lse<T, true, kGrpThreads>(row, lo, hi, a.k2, s_c, s_z, C, Z);
    if (wave == 0) {
      if (lane == 0) {
        unsigned long long* rec = a.pchunk + static_cast<size_t>(blockIdx.x) * 4;
        store_sys(rec + 0, rec_word(C, a.ptag));
        store_sys(rec + 1, rec_word(Z, a.ptag));
        store_sys(rec + 2, rec_word(lx, a.ptag));
        store_sys(rec + 3, rec_word(qx, a.ptag));
      }
      // the sequence's records, record l in lane l; then lane i merges row i's chunks
      const unsigned long long* rb = a.pchunk + static_cast<size_t>(b) * W * 4;
      const bool live = lane < W;
      unsigned long long r0 = 0, r1 = 0, r2 = 0, r3 = 0;
      for (int polls = 0;; ++polls) {
        if (live) {
          r0 = load_sys(rb + lane * 4);
          r1 = load_sys(rb + lane * 4 + 1);
          r2 = load_sys(rb + lane * 4 + 2);
          r3 = load_sys(rb + lane * 4 + 3);
        }
        const bool ok = !live || (rec_tagged(r0, a.ptag) && rec_tagged(r1, a.ptag) && rec_tagged(r2, a.ptag) &&
                                  rec_tagged(r3, a.ptag));
        if (__ballot(!ok) == 0) break;
        if (polls >= kGrpSpinCap) {
          if (lane == 0) atomicOr(a.err, SV_DATA_STALL);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      const float Cl = rec_value(r0), Zl = rec_value(r1), lxl = rec_value(r2), qxl = rec_value(r3);
      float Cm = -FLT_MAX, Zm = 0.f;
      for (int kk = 0; kk < S; ++kk) {  // chunk order, the same in every workgroup and call
        const float c2 = __shfl(Cl, ii * S + kk), z2 = __shfl(Zl, ii * S + kk);
        lse2_merge(Cm, Zm, c2, z2);
      }
      const int kx = xv >= 0 && xv < V ? min(xv / a.span, S - 1) : 0;
      const float lxv = __shfl(lxl, ii * S + kx), qxv = __shfl(qxl, ii * S + kx);
      bool acc = true;
      if (lane < g) {
        double px;
        const bool mine = lane == i && k == 0;  // one workgroup flags and reports row i
        acc = accept_decision(xv, lxv, qxv, uu, Cm, Zm, a, px, mine);
        if (mine && a.pdraft) a.pdraft[base + lane] = static_cast<float>(px);
      }
      const unsigned long long rej = __ballot(lane < g && !acc);
      const int n = rej ? __ffsll(rej) - 1 : g;
      const int src = n < g ? n : 0;
      const float cr = __shfl(Cm, src), zr = __shfl(Zm, src);
      const int xn = __shfl(xv, src);
      if (lane == 0)
        s_d = GroupDraw{n < g ? static_cast<double>(zr) : 0.0, n < g ? draw_ref(a, cr) : 0.0, n, g, base,
                        n < g ? xn : -1, b, uf};
    }
  } else if (threadIdx.x == 0) {
    s_d = GroupDraw{0.0, 0.0, 0, 0, 0, -1, b, a.u[b]};
  }
  __syncthreads();  // s_d, s_tab
  const GroupDraw dd = uniform_draw(s_d);
  const int unit = j * kGrpWaves + wave;
  if (unit >= a.nunits) return;
  const T* lrow = drawn_row<T>(a, dd);
  const float* qrow = drawn_q(a, dd);
  const bool residual = dd.n < dd.g;
  const int r0 = unit * a.uw, r1 = min(V, r0 + a.uw);
  double D, Q, Zs;
  draw_sweep<T, true>(lrow, qrow, r0, r1, kExpScale * a.k2d, kExpScale * (residual ? dd.cr : 0.0),
                      residual ? dd.zr : 0.0, s_tab, D, Q, Zs);
  // the unit's three sums as six tagged words (each 32-bit half with the call's tag)
  unsigned long long* sums = a.psum + static_cast<size_t>(b) * kGrpMaxUnits * kSumWords;
  if (lane == 0) {
    unsigned long long* dst = sums + static_cast<size_t>(unit) * kSumWords;
    const double v[3] = {D, Q, Zs};
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const unsigned long long x = static_cast<unsigned long long>(__double_as_longlong(v[t]));
      store_sys(dst + 2 * t, (x & 0xFFFFFFFF00000000ull) | a.ptag);
      store_sys(dst + 2 * t + 1, (x << 32) | a.ptag);
    }
  }
  if (unit != 0) return;
  // the finisher (unit 0's wave): every unit's sums, unit u in lane u
  const bool live = lane < a.nunits;
  const unsigned long long* src = sums + static_cast<size_t>(live ? lane : 0) * kSumWords;
  unsigned long long w[kSumWords];
  for (int polls = 0;; ++polls) {
    bool ok = true;
#pragma unroll
    for (int t = 0; t < kSumWords; ++t) {
      w[t] = live ? load_sys(src + t) : 0ull;
      ok = ok && (!live || rec_tagged(w[t], a.ptag));
    }
    if (__ballot(!ok) == 0) break;
    if (polls >= kGrpSpinCap) {
      if (lane == 0) atomicOr(a.err, SV_DATA_STALL);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  double v[3];
#pragma unroll
  for (int t = 0; t < 3; ++t)
    v[t] = live ? __longlong_as_double(static_cast<long long>((w[2 * t] & 0xFFFFFFFF00000000ull) | (w[2 * t + 1] >> 32)))
                : 0.0;
  group_finish<T>(a, dd, v[0], v[1], v[2], s_tab, xv);
}

// ---- short rows: one workgroup per sequence
// With rows of at most kTinyMaxV entries one workgroup takes a whole sequence and every
// hand-off goes through LDS: wave w computes the softmax state of draft rows w, w + 8, ...
// (the draft's logit and q entry loaded ahead of the row), wave 0 runs the accept tests of
// all rows, the waves sweep one unit each of the drawn row, and wave 0 finishes the draw.
constexpr int kTinyMaxV = 4096;

template <typename T>
__global__ __launch_bounds__(kGrpThreads) void k_verify_tiny(Args a) {
  __shared__ double s_tab[kExpN];
  __shared__ float s_rc[kFuseMaxGamma], s_rz[kFuseMaxGamma], s_lx[kFuseMaxGamma], s_qx[kFuseMaxGamma];
  __shared__ double s_us[kGrpWaves][3];
  __shared__ GroupDraw s_d;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int V = a.V, g = a.gamma, b = static_cast<int>(blockIdx.x), base = b * g;
  exp_table_init(s_tab);
  int xv = 0;
  float uu = 0.f, uf = 0.f;
  if (wave == 0) {  // drafts and uniforms of the sequence (lane i: row i)
    if (g > 0) {
      const int ii = min(lane, g - 1);
      xv = a.ids[base + ii];
      uu = a.u[base + ii + b];
    }
    uf = a.u[base + b + g];
  }
  for (int i = wave; i < g; i += kGrpWaves) {
    const int d = base + i;
    const T* row = static_cast<const T*>(a.logits) + static_cast<size_t>(d + b) * V;
    float lx = 0.f, qx = 0.f;
    if (lane == 0) {
      const int x = a.ids[d];
      if (x >= 0 && x < V) {
        lx = load_one(row, x);
        qx = a.onehot ? 1.f : a.q[static_cast<size_t>(d) * V + x];
      }
    }
    float c, z;
    wave_row_lse<T, true, 64>(row, 0, V, a.k2, lane, c, z);
    if (lane == 0) {
      s_rc[i] = c;
      s_rz[i] = z;
      s_lx[i] = lx;
      s_qx[i] = qx;
    }
  }
  __syncthreads();  // s_rc, s_rz, s_lx, s_qx, s_tab
  if (wave == 0) {
    bool acc = true;
    float Cm = 0.f, Zm = 0.f;
    if (lane < g) {
      double px;
      Cm = s_rc[lane];
      Zm = s_rz[lane];
      acc = accept_decision(xv, s_lx[lane], s_qx[lane], uu, Cm, Zm, a, px, true);
      if (a.pdraft) a.pdraft[base + lane] = static_cast<float>(px);
    }
    const unsigned long long rej = __ballot(lane < g && !acc);
    const int n = rej ? __ffsll(rej) - 1 : g;
    const int src = n < g ? n : 0;
    const float cr = __shfl(Cm, src), zr = __shfl(Zm, src);
    const int xn = __shfl(xv, src);
    if (lane == 0)
      s_d = GroupDraw{n < g ? static_cast<double>(zr) : 0.0, n < g ? draw_ref(a, cr) : 0.0, n, g, base,
                      n < g ? xn : -1, b, uf};
  }
  __syncthreads();  // s_d
  const GroupDraw dd = uniform_draw(s_d);
  if (wave < a.nunits) {
    const bool residual = dd.n < dd.g;
    const int r0 = wave * a.uw, r1 = min(V, r0 + a.uw);
    double D, Q, Zs;
    draw_sweep<T, true>(drawn_row<T>(a, dd), drawn_q(a, dd), r0, r1, kExpScale * a.k2d,
                        kExpScale * (residual ? dd.cr : 0.0), residual ? dd.zr : 0.0, s_tab, D, Q, Zs);
    if (lane == 0) {
      s_us[wave][0] = D;
      s_us[wave][1] = Q;
      s_us[wave][2] = Zs;
    }
  }
  __syncthreads();  // s_us
  if (wave == 0) {
    const bool live = lane < a.nunits;
    group_finish<T>(a, dd, live ? s_us[lane][0] : 0.0, live ? s_us[lane][1] : 0.0, live ? s_us[lane][2] : 0.0,
                    s_tab, xv);
  }
}

// The judged rows are read with ordinary loads: nontemporal ones measured slower on
// MI355X with inputs rotated past the last-level cache (B = 256, gamma = 4, V = 128256
// bf16: 70.1 against 69.5 us; B = 160: 59.4 against 59.1 us).
template <typename T, bool RAGGED>
__global__ __launch_bounds__(kSeqThreads) void k_verify_seq(Args a) {
  __shared__ double s_tab[kExpN];
  __shared__ float2 s_cz[kFuseMaxGamma];
  __shared__ int s_xn;
  const int b = RAGGED && a.order ? a.order[blockIdx.x] : blockIdx.x;
  int base, g;
  if (!seq_geom<RAGGED>(a, b, base, g)) {
    if (threadIdx.x == 0) {
      atomicOr(a.err, SV_DATA_CU_GAMMA);
      a.acc[b] = -1;
    }
    return;
  }
  if constexpr (sizeof(T) == 2) {
    __shared__ double sT[kTabEntries];
    const bool tab = a.tlo <= a.thi;
    if (!tab) exp_table_init(s_tab);  // with the table, only the fallback draw needs it
    // the value table is built while the first loads of pass 1 are in flight
    auto hook = [&] {
      if (tab) tab_build(sT, a);
    };
    const int n = g == 0 ? 0
                  : a.V >= kSeqWaves * kIter ? judge_rows_exact<T, true, false>(a, b, base, g, s_cz, &s_xn, hook)
                                             : judge_rows_exact<T, false, false>(a, b, base, g, s_cz, &s_xn, hook);
    if (g == 0) {
      if (tab) tab_build(sT, a);
      if (threadIdx.x == 0) a.acc[b] = 0;
    }
    __syncthreads();  // s_cz of row n, sT (s_tab without the table)
    const double cr = n < g ? draw_ref(a, s_cz[n].x) : 0.0;
    const double zr = n < g ? static_cast<double>(s_cz[n].y) : 0.0;
    // table scale: sum 2^(l k2) = z 2^c
    const int xn = n < g ? s_xn : -1;
    if (tab && final_draw_tab(a, b, base, g, n, zr * exp2(cr), sT, xn)) return;
    if (tab) {
      exp_table_init(s_tab);
      __syncthreads();  // s_tab
    }
    final_draw<T, true>(a, b, base, g, n, cr, zr, s_tab, xn);
  } else {
    exp_table_init(s_tab);
    const int n = g == 0 ? 0
                  : a.V >= kSeqWaves * kIter ? judge_rows_exact<T, true, false>(a, b, base, g, s_cz, &s_xn, [] {})
                                             : judge_rows_exact<T, false, false>(a, b, base, g, s_cz, &s_xn, [] {});
    if (g == 0 && threadIdx.x == 0) a.acc[b] = 0;
    __syncthreads();  // s_cz of row n, s_tab
    final_draw<T, true>(a, b, base, g, n, n < g ? draw_ref(a, s_cz[n].x) : 0.0,
                        n < g ? static_cast<double>(s_cz[n].y) : 0.0, s_tab, n < g ? s_xn : -1);
  }
}

// ---- the row kernel's two teams: the 16 waves form two teams of eight, each drawing its
// own rows, so that one team's finish (search and re-sweep, bound by latency) overlaps
// the other team's sweep (bound by HBM). A team meets at team barriers: each wave adds
// one to its team's LDS counter, then polls it until the whole team has arrived. Every
// poll loop is bounded: past kSpinCap polls the wave raises SV_DATA_STALL and goes on,
// so no wave waits without end.
constexpr int kTeams = 2;
constexpr int kTeamWaves = kSeqWaves / kTeams;
constexpr int kTeamPass = kTeamWaves * kIter;  // entries a team re-sweeps per pass
constexpr int kSpinCap = 1 << 22;
static_assert(kSeqWaves % kTeams == 0, "teams of equal size");

// `target` counts the arrivals this wave has waited for so far (the same in every wave
// of the team).
__device__ __forceinline__ void team_barrier(int* cnt, int& target, int* err) {
  target += kTeamWaves;
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");  // this wave's writes are done
  if ((threadIdx.x & 63) == 0) atomicAdd(cnt, 1);
  int polls = 0;
  while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
    if (++polls > kSpinCap) {
      if ((threadIdx.x & 63) == 0) atomicOr(err, SV_DATA_STALL);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
}

// A team's finish of row b drawn from p (gamma = 0): lane k < kSeqWaves of every wave of
// the team holds the table sum of sub-region k (width sw); the same search as tab_finish
// (t = u Z, the sub-region where the inclusive prefix first exceeds t, else the last
// positive one), then the team re-sweeps that sub-region in passes of kTeamPass entries
// for the first entry whose prefix exceeds t. Writes emitted[b] and residual_sum[b] = 0.
// Ends with a team barrier, after which the team's LDS may be reused.
__device__ __forceinline__ void team_finish(const Args& a, int b, const double* sT, double rD, int sw, int tw,
                                            double (*s_wt)[kTeamWaves], int* s_cand, int* s_last, int* cnt,
                                            int& target, float uf) {
  const int lane = threadIdx.x & 63;
  const int V = a.V;
  const int tlo = a.tlo, tsent = a.thi + 1 - a.tlo;
  const uint16_t* lrow = drawn_row(a, b, 0, 0, 0);
  const bool live = lane < kSeqWaves;
  const double wgt = live ? rD : 0.0;
  const double Z64 = wave_sum_dpp(wgt);
  const double t = static_cast<double>(uf) * Z64;
  const double inc = wave_incl_scan_dpp(wgt);
  const unsigned long long cross = __ballot(live && inc > t);
  int rs = cross ? __ffsll(cross) - 1 : -1;
  double run = readlane_d(inc - wgt, rs < 0 ? 0 : rs);
  bool take_last = false;
  if (rs < 0) {  // no crossing (rounding, or u >= 1): last positive-weight entry
    take_last = true;
    const unsigned long long pos = __ballot(live && wgt > 0.0);
    rs = pos ? 63 - __clzll(pos) : -1;
    run = 0.0;
  }
  if (tw == 0 && lane == 0) {
    if (!(Z64 > 0.0 && Z64 <= DBL_MAX)) atomicOr(a.err, SV_DATA_NONFINITE);
    if (!(uf >= 0.f && uf < 1.f)) atomicOr(a.err, SV_DATA_UNIFORM);
    *s_cand = INT_MAX;
    *s_last = -1;
  }
  int tok = V - 1;
  if (rs >= 0) {
    const int R0 = min(V, rs * sw), R1 = min(V, R0 + sw);
    int parity = 0;
    for (int p0 = R0; p0 < R1; p0 += kTeamPass, parity ^= 1) {
      const int e = p0 + tw * kIter + lane * kGroup;
      const bool in = e < R1;
      Raw<uint16_t> lr;
      load_raw_in(lrow, min(e, R1 - kGroup), lr);
      double rv[kGroup];
      lookup8(lr, rv, sT, tlo, tsent);
      double tot = 0.0;
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        rv[j] = in ? rv[j] : 0.0;
        tot += rv[j];
      }
      const double linc = wave_incl_scan_dpp(tot);
      if (lane == 63) s_wt[parity][tw] = linc;
      team_barrier(cnt, target, a.err);
      double acc = run, tsum = run;
      for (int w2 = 0; w2 < kTeamWaves; ++w2) {
        const double v2 = s_wt[parity][w2];
        if (w2 < tw) acc += v2;
        tsum += v2;
      }
      acc += linc - tot;
      int c2 = INT_MAX, lp = -1;
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        acc += rv[j];
        if (!take_last && c2 == INT_MAX && acc > t) c2 = e + j;
        if (rv[j] > 0.0) lp = e + j;
      }
      c2 = wave_min_int_dpp(c2);
      lp = wave_max_int_dpp(lp);
      if (lane == 0) {
        if (c2 != INT_MAX) atomicMin(s_cand, c2);
        if (lp >= 0) atomicMax(s_last, lp);
      }
      run = tsum;
      team_barrier(cnt, target, a.err);
      if (*s_cand != INT_MAX) break;
    }
    tok = *s_cand != INT_MAX ? *s_cand : (*s_last >= 0 ? *s_last : V - 1);
  }
  if (tw == 0 && lane == 0) {
    a.emitted[b] = tok;
    a.rsum[b] = 0.f;
  }
  team_barrier(cnt, target, a.err);  // s_cand, s_last and the sums are read
}

// Rounds with no drafts (gamma = 0: one token per row drawn from p, [P1] ch.2 bonus draw)
// with more rows than compute units: one workgroup per compute unit builds the value
// table once and draws row after row (rows b, b + gridDim.x, ...), instead of one
// workgroup, and one table, per row. bf16 rows: two teams of eight waves take
// alternate rows (team_finish); a row holding a value outside the table is marked and
// drawn afterwards by the whole workgroup on the exp2 path.
constexpr int kFallbackMark = -2;  // emitted[b] of a row left for the exp2 path
template <typename T>
__global__ __launch_bounds__(kSeqThreads) void k_sample_rows(Args a) {
  __shared__ double s_tab[kExpN];
  if constexpr (sizeof(T) == 2) {
    __shared__ double sT[kTabEntries];
    __shared__ double s_rs[kTeams][kSeqWaves];          // a team's sub-region sums of its row
    __shared__ double s_wt[kTeams][2][kTeamWaves];      // re-sweep: per-wave totals, by pass parity
    __shared__ int s_cand[kTeams], s_last[kTeams], s_cnt[kTeams];
    __shared__ int s_fb, s_nfb;
    const bool tab = a.tlo <= a.thi;
    if (!tab) {
      exp_table_init(s_tab);
      __syncthreads();  // s_tab
      for (int b = blockIdx.x; b < a.B; b += gridDim.x) {
        if (threadIdx.x == 0) a.acc[b] = 0;
        final_draw<T, true>(a, b, 0, 0, 0, 0.0, 0.0, s_tab);
        __syncthreads();  // the draw's LDS is reused by the next row
      }
      return;
    }
    tab_build(sT, a);
    if (threadIdx.x < kTeams) s_cnt[threadIdx.x] = 0;
    if (threadIdx.x == 0) s_nfb = 0;
    __syncthreads();  // sT, s_cnt, s_nfb
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int team = wave / kTeamWaves, tw = wave % kTeamWaves;
    const int V = a.V;
    const int sw = sub_width(V, kSeqWaves);
    int target = 0;
    for (int b = blockIdx.x + team * gridDim.x; b < a.B; b += kTeams * gridDim.x) {
      if (tw == 0 && lane == 0) a.acc[b] = 0;
      const float uf = a.u[b];  // loaded before the sweep, used after it
      // this wave's two sub-regions of the row: tw and tw + kTeamWaves
#pragma unroll
      for (int h = 0; h < kTeams; ++h) {
        const int k = tw + h * kTeamWaves;
        const int r0 = min(V, k * sw), r1 = min(V, r0 + sw);
        double D, Q, Z;
        tab_sweep(drawn_row(a, b, 0, 0, 0), nullptr, r0, r1, 0.0, sT, a.tlo, a.thi + 1 - a.tlo, D, Q, Z);
        if (lane == 0) s_rs[team][k] = D;
      }
      team_barrier(&s_cnt[team], target, a.err);  // s_rs[team]
      const double rD = s_rs[team][lane < kSeqWaves ? lane : 0];
      // a value outside the table reached the sentinel: a sub-region sum is not finite
      if (__ballot(lane < kSeqWaves && !(rD <= DBL_MAX)) != 0) {
        if (tw == 0 && lane == 0) {
          a.emitted[b] = kFallbackMark;
          atomicAdd(&s_nfb, 1);
        }
        team_barrier(&s_cnt[team], target, a.err);  // s_rs[team] is read
        continue;
      }
      team_finish(a, b, sT, rD, sw, tw, s_wt[team], &s_cand[team], &s_last[team], &s_cnt[team], target, uf);
    }
    __syncthreads();  // both teams are done; marked rows are visible to the workgroup
    if (s_nfb == 0) return;
    bool exp_ready = false;
    for (int b = blockIdx.x; b < a.B; b += gridDim.x) {
      if (threadIdx.x == 0) s_fb = a.emitted[b] == kFallbackMark;
      __syncthreads();  // s_fb
      const bool fb = s_fb;
      __syncthreads();  // s_fb is read before the next row rewrites it
      if (!fb) continue;
      if (!exp_ready) {
        exp_table_init(s_tab);
        __syncthreads();  // s_tab
        exp_ready = true;
      }
      final_draw<T, true>(a, b, 0, 0, 0, 0.0, 0.0, s_tab);
      __syncthreads();  // the draw's LDS is reused by the next row
    }
  } else {
    exp_table_init(s_tab);
    __syncthreads();  // s_tab
    for (int b = blockIdx.x; b < a.B; b += gridDim.x) {
      if (threadIdx.x == 0) a.acc[b] = 0;
      final_draw<T, true>(a, b, 0, 0, 0, 0.0, 0.0, s_tab);
      __syncthreads();
    }
  }
}

// Greedy in one launch ([P1] ch.3 greedy; [P4] "출력이 변하지 않는다는 것이 핵심이다"): one
// workgroup per sequence walks rows 0..g through the same register ring as the sampling
// path and takes each row's argmax (largest value, lowest index); draft i is accepted iff
// it equals the argmax of row i. The walk stops at the first mismatch, whose argmax is the
// emitted token, or after the bonus row g. Rows after the mismatch are not read.
template <typename T, bool RAGGED, bool NT1>
__global__ __launch_bounds__(kSeqThreads) void k_greedy_seq1(Args a) {
  __shared__ float s_v[kSeqWaves];
  __shared__ int s_i[kSeqWaves];
  const int b = RAGGED && a.order ? a.order[blockIdx.x] : blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int base, g;
  if (!seq_geom<RAGGED>(a, b, base, g)) {
    if (threadIdx.x == 0) {
      atomicOr(a.err, SV_DATA_CU_GAMMA);
      a.acc[b] = -1;
    }
    return;
  }
  const int V = a.V;
  const T* Lseq = static_cast<const T*>(a.logits) + static_cast<size_t>(base + b) * V;
  const int x = g > 0 ? a.ids[base + min(lane, g - 1)] : -1;  // lane i: draft i
  constexpr int kSpan = kSeqWaves * kIter;
  const int lane_off = wave * kIter + lane * kGroup;
  const int nsp = (V + kSpan - 1) / kSpan;
  const bool wide = V >= kSpan;
  // index of this lane's first entry in span k, matching walk_rows' loads
  auto entry0 = [&](int k) {
    return wide ? (k < nsp - 1 ? k * kSpan : V - kSpan) + lane_off : min(lane_off, V - kGroup);
  };
  float bv = -INFINITY;
  float nw = -INFINITY;  // NaN watch of the row
  int bi = entry0(0);  // a row of -inf still yields its lowest index
  int n = g, tok = -1;
  auto step = [&](const Raw<T>& lr, int k) {
    float xv[kGroup];
    unpack(lr, xv);
    nw = nan_watch(nw, xv);
    const int e = entry0(k);
#pragma unroll
    for (int j = 0; j < kGroup; ++j)
      if (xv[j] > bv) {  // strict: a lane visits its entries in increasing index order
        bv = xv[j];
        bi = e + j;
      }
  };
  auto row_end = [&](int i) -> bool {
    // a NaN in a judged row is a data error; the argmax is then unspecified
    flag_nan(nw, a.err, SV_DATA_NONFINITE);
    nw = -INFINITY;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float v2 = __shfl_xor(bv, o);
      const int i2 = __shfl_xor(bi, o);
      argmax_merge(bv, bi, v2, i2);
    }
    if (lane == 0) {
      s_v[wave] = bv;
      s_i[wave] = bi;
    }
    __syncthreads();
    // every wave merges the 16 partials in the same order and takes the same decision
    float Vm = s_v[0];
    int I = s_i[0];
    for (int w = 1; w < kSeqWaves; ++w) argmax_merge(Vm, I, s_v[w], s_i[w]);
    bv = -INFINITY;
    bi = entry0(0);
    __syncthreads();  // s_v / s_i are rewritten by the next row
    if (i == g) {  // the bonus row
      tok = I;
      return true;
    }
    const int xi = __shfl(x, i);
    if (wave == 0 && lane == 0 && bad_id(a, xi)) atomicOr(a.err, SV_DATA_DRAFT_ID);
    if (xi != I) {
      n = i;
      tok = I;
      return true;
    }
    return false;
  };
  if (wide)
    walk_rows<T, true, NT1>(Lseq, V, g + 1, [] {}, step, row_end);
  else
    walk_rows<T, false, NT1>(Lseq, V, g + 1, [] {}, step, row_end);
  if (wave == 0) {
    if (lane < n) a.emitted[base + b + lane] = x;
    if (lane == 0) {
      a.acc[b] = n;
      a.emitted[base + b + n] = tok;
      a.rsum[b] = 0.f;
    }
  }
  for (int i = n + 1 + threadIdx.x; i <= g; i += kSeqThreads) a.emitted[base + b + i] = -1;
}

// One participant's part of a greedy sequence with helpers (k_greedy_help): walks the
// rows it claims from the sequence's counter, starting with r0 and r1 (claimed ahead so
// the next row's first loads overlap the row being read), publishes a mismatch (or the
// bonus row's argmax) with an atomic min of (row, argmax), stops at a row past g or past
// the smallest published row, then leaves; the participant that brings the count to zero
// writes the outputs. Every thread of the block calls it.
template <typename T>
__device__ __forceinline__ void greedy_participate(const Args& a, int b, int base, int g, int r0, int r1) {
  __shared__ float s_v[kSeqWaves];
  __shared__ int s_i[kSeqWaves];
  __shared__ int s_ctl[2];
  __shared__ int s_out[3];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  unsigned long long* claim = a.gclaim + b;
  unsigned long long* part = a.gpart + b;
  unsigned long long* best = a.gbest + b;
  const int V = a.V;
  const T* L0 = static_cast<const T*>(a.logits) + static_cast<size_t>(base + b) * V;
  const int x = g > 0 ? a.ids[base + min(lane, g - 1)] : -1;  // lane i: draft i
  constexpr int kSpan = kSeqWaves * kIter;
  const int lane_off = wave * kIter + lane * kGroup;
  const int nsp = (V + kSpan - 1) / kSpan;
  const bool wide = V >= kSpan;
  auto entry0 = [&](int k) {
    return wide ? (k < nsp - 1 ? k * kSpan : V - kSpan) + lane_off : min(lane_off, V - kGroup);
  };
  // walked row t is row rc, walked row t + 1 is row rn (both the same in every thread)
  int tw = 0, rc = r0, rn = r1;
  auto row_ptr = [&](int il) {
    const int r = min(il == tw ? rc : rn, g);  // a claim past g reads row g, never judged
    return L0 + static_cast<size_t>(r) * V;
  };
  float bv = -INFINITY;
  float nw = -INFINITY;  // NaN watch of the row
  int bi = entry0(0);
  auto step = [&](const Raw<T>& lr, int k) {
    float xv[kGroup];
    unpack(lr, xv);
    nw = nan_watch(nw, xv);
    const int e = entry0(k);
#pragma unroll
    for (int q = 0; q < kGroup; ++q)
      if (xv[q] > bv) {
        bv = xv[q];
        bi = e + q;
      }
  };
  auto row_end = [&](int t) -> bool {
    const int i = rc;  // the row just read
    flag_nan(nw, a.err, SV_DATA_NONFINITE);  // a NaN in a row this participant judged
    nw = -INFINITY;
    // the next claim and the published minimum, loaded now so the merge hides them
    unsigned long long nc = 0, nb = ~0ull;
    if (threadIdx.x == 0) {
      nc = __hip_atomic_fetch_add(claim, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      nb = __hip_atomic_load(best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float v2 = __shfl_xor(bv, o);
      const int i2 = __shfl_xor(bi, o);
      argmax_merge(bv, bi, v2, i2);
    }
    if (lane == 0) {
      s_v[wave] = bv;
      s_i[wave] = bi;
    }
    __syncthreads();
    float Vm = s_v[0];
    int I = s_i[0];
    for (int w = 1; w < kSeqWaves; ++w) argmax_merge(Vm, I, s_v[w], s_i[w]);
    bv = -INFINITY;
    bi = entry0(0);
    const bool stop = i == g || __shfl(x, i < g ? i : 0) != I;  // the bonus row, or a mismatch
    if (threadIdx.x == 0) {
      if (stop) {
        const unsigned long long mine = (static_cast<unsigned long long>(i) << 32) | static_cast<uint32_t>(I);
        (void)__hip_atomic_fetch_min(best, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      }
      s_ctl[0] = static_cast<int>(static_cast<uint32_t>(nc));
      s_ctl[1] = static_cast<int>(min(nb >> 32, 0x7FFFFFFFull));
    }
    __syncthreads();  // s_v / s_i are rewritten by the next row; s_ctl is read
    const int next = s_ctl[0], known = s_ctl[1];
    __syncthreads();  // s_ctl is rewritten by the next row
    if (stop || rn > g || known < rn) return true;
    tw = t + 1;
    rc = rn;
    rn = next;
    return false;
  };
  if (r0 <= g) {
    if (wide)
      walk_rows_p<T, true, false>(row_ptr, V, g + 1, [] {}, step, row_end);
    else
      walk_rows_p<T, false, false>(row_ptr, V, g + 1, [] {}, step, row_end);
  }
  // leave; the participant that brings the count to zero writes the outputs
  if (threadIdx.x == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the published minimum first
    const unsigned long long p = __hip_atomic_fetch_sub(part, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    s_out[2] = static_cast<uint32_t>(p) == 1u ? 1 : 0;
    if (s_out[2]) {
      const unsigned long long m = __hip_atomic_load(best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      const int nr = static_cast<int>(min(m >> 32, static_cast<unsigned long long>(g)));
      s_out[0] = nr;
      s_out[1] = static_cast<int>(static_cast<uint32_t>(m));
      if (nr < g && bad_id(a, a.ids[base + nr])) atomicOr(a.err, SV_DATA_DRAFT_ID);
    }
  }
  __syncthreads();
  const bool writer = s_out[2] != 0;
  const int n = s_out[0], tok = s_out[1];
  __syncthreads();  // s_out is rewritten by a helper's next sequence
  if (!writer) return;
  if (wave == 0) {
    if (lane < n) a.emitted[base + b + lane] = x;
    if (lane == 0) {
      a.acc[b] = n;
      a.emitted[base + b + n] = tok;
      a.rsum[b] = 0.f;
    }
  }
  for (int i = n + 1 + threadIdx.x; i <= g; i += kSeqThreads) a.emitted[base + b + i] = -1;
}

// Greedy in one launch with helpers: workgroups 0..B-1 own one sequence each, as in
// k_greedy_seq1; workgroup B + h is a helper, dispatched only as the owners' slots free
// up, that joins sequence h (in the same order as the owners) if it still has rows to
// claim and no mismatch has been published (otherwise every new claim would lie past
// it), takes part as in greedy_participate and exits. Row n, the first mismatch, is
// always claimed before any row after it and judged by its claimer, so the minimum holds
// it when the last participant leaves. Counters carry the call's epoch, so no reset is
// needed; nothing waits for another workgroup, and all of it is kept past the per-XCD L2
// caches (system scope).
template <typename T, bool RAGGED>
__global__ __launch_bounds__(kSeqThreads) void k_greedy_help(Args a) {
  __shared__ int s_join[3];
  const bool helper = blockIdx.x >= static_cast<unsigned>(a.B);
  const int bi0 = static_cast<int>(blockIdx.x % static_cast<unsigned>(a.B));
  const int b = RAGGED && a.order ? a.order[bi0] : bi0;
  int base, g;
  if (!seq_geom<RAGGED>(a, b, base, g)) {
    if (!helper && threadIdx.x == 0) {
      atomicOr(a.err, SV_DATA_CU_GAMMA);
      a.acc[b] = -1;
    }
    return;
  }
  const unsigned long long E = static_cast<unsigned long long>(a.gepoch) << 32;
  unsigned long long* claim = a.gclaim + b;
  unsigned long long* part = a.gpart + b;
  unsigned long long* best = a.gbest + b;
  if (threadIdx.x == 0) {
    int r0 = 0, r1 = 1;
    if (!helper) {  // fresh state for this call; rows 0 and 1 are the owner's
      __hip_atomic_store(best, ~0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      __hip_atomic_store(part, E | 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // before the counter shows this epoch
      __hip_atomic_store(claim, E | 2ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    } else {
      const unsigned long long c = __hip_atomic_load(claim, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      const bool join = (c >> 32) == a.gepoch && static_cast<uint32_t>(c) <= static_cast<uint32_t>(g) &&
                        __hip_atomic_load(best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == ~0ull;
      r0 = r1 = INT_MAX;
      if (join) {
        (void)__hip_atomic_fetch_add(part, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // counted before claiming
        r0 = static_cast<int>(static_cast<uint32_t>(
            __hip_atomic_fetch_add(claim, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM)));
        r1 = static_cast<int>(static_cast<uint32_t>(
            __hip_atomic_fetch_add(claim, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM)));
      }
      s_join[0] = join ? 1 : 0;
    }
    s_join[1] = r0;
    s_join[2] = r1;
  }
  __syncthreads();
  if (helper && !s_join[0]) return;  // a helper that did not join leaves nothing behind
  greedy_participate<T>(a, b, base, g, s_join[1], s_join[2]);
}

// ============================================================== sampling from given weights
// One token per row from weights w >= 0 (fp32, normalised or not): the inverse CDF of
// the draw ([P1] ch.2; [P3] 단계 1 draws the drafts from q), t = u sum(w), the first v
// whose inclusive prefix exceeds t, else the last v with positive weight. Negative or
// non-finite weights count as 0 and raise the non-finite flag. One 1024-thread
// workgroup per row: a sweep of region sums in fp64 (wave w owns region w), every
// wave's search over the 16 sums, a re-sweep of the crossing region.
template <bool ALIGNED>
__global__ __launch_bounds__(kSeqThreads) void k_sample_weights(const float* __restrict__ w, const float* u,
                                                               int32_t* tokens, int* err, int V) {
  __shared__ double s_reg[kSeqWaves];
  __shared__ double s_wt[2][kSeqWaves];
  __shared__ int s_cand, s_last, s_bad;
  const int row = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (threadIdx.x == 0) {
    s_cand = INT_MAX;
    s_last = -1;
    s_bad = 0;
  }
  const float* wrow = w + static_cast<size_t>(row) * V;
  const int rw = region_width(V);
  const int r0 = min(V, wave * rw), r1 = min(V, r0 + rw);
  const int nfull = ALIGNED ? (r1 - r0) / kIter : 0;
  const int mstart = r0 + nfull * kIter;
  double acc = 0.0;
  bool bad = false;
  auto step = [&](const Raw<float>& r) {
    float v[kGroup];
    unpack(r, v);
    double s0 = 0.0, s1 = 0.0;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      bad |= !(v[j] >= 0.f && v[j] <= FLT_MAX);
      const double c = fmax(static_cast<double>(v[j]), 0.0);  // NaN -> 0
      if (j & 1) s1 += c; else s0 += c;
    }
    acc += s0 + s1;
  };
  if (nfull > 0) {
    Raw<float> Lb[kRing];
    const int eb = r0 + lane * kGroup, last = nfull - 1;
    auto at = [&](int it) { return eb + min(it, last) * kIter; };
#pragma unroll
    for (int k = 0; k < kRing - 1; ++k) {
      load_raw_in(wrow, at(k), Lb[k]);
      issue_order_fence();
    }
    for (int it = 0; it < nfull; it += kRing) {
#pragma unroll
      for (int k = 0; k < kRing; ++k) {
        load_raw_in(wrow, at(it + k + kRing - 1), Lb[(k + kRing - 1) % kRing]);
        if (k == 0 || it + k < nfull) step(Lb[k]);
      }
    }
  }
  for (int e0 = mstart; e0 < r1; e0 += kIter) {  // the rest of the region, 0 past r1
    Raw<float> r;
    load_raw<float, ALIGNED>(wrow, e0 + lane * kGroup, r1, r, 0u);
    step(r);
  }
  acc = wave_sum_dpp(acc);
  if (lane == 0) s_reg[wave] = acc;
  if (__ballot(bad) != 0 && lane == 0) atomicOr(&s_bad, 1);
  __syncthreads();
  const float uf = u[row];
  const bool live = lane < kSeqWaves;
  const double wgt = live ? s_reg[lane] : 0.0;
  const double tot = wave_sum_dpp(wgt);
  const double t = static_cast<double>(uf) * tot;
  const double inc = wave_incl_scan_dpp(wgt);
  const unsigned long long cross = __ballot(live && inc > t);
  int rs = cross ? __ffsll(cross) - 1 : -1;
  double run = readlane_d(inc - wgt, rs < 0 ? 0 : rs);
  bool take_last = false;
  if (rs < 0) {
    take_last = true;
    const unsigned long long pos = __ballot(live && wgt > 0.0);
    rs = pos ? 63 - __clzll(pos) : -1;
    run = 0.0;
  }
  if (threadIdx.x == 0) {
    if (s_bad || !(tot > 0.0 && tot <= DBL_MAX)) atomicOr(err, SV_DATA_NONFINITE);
    if (!(uf >= 0.f && uf < 1.f)) atomicOr(err, SV_DATA_UNIFORM);
  }
  int tok = V - 1;
  if (rs >= 0) {
    const int R0 = min(V, rs * rw), R1 = min(V, R0 + rw);
    int parity = 0;
    for (int p0 = R0; p0 < R1; p0 += kPass, parity ^= 1) {
      const int e = p0 + wave * kIter + lane * kGroup;
      Raw<float> r;
      load_raw<float, ALIGNED>(wrow, e, R1, r, 0u);
      float v[kGroup];
      unpack(r, v);
      double rv[kGroup];
      double tsum_l = 0.0;
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        rv[j] = fmax(static_cast<double>(v[j]), 0.0);
        tsum_l += rv[j];
      }
      const double linc = wave_incl_scan_dpp(tsum_l);
      const double lex = linc - tsum_l;
      if (lane == 63) s_wt[parity][wave] = linc;
      __syncthreads();
      double accp = run, tsum = run;
      for (int w2 = 0; w2 < kSeqWaves; ++w2) {
        const double v2 = s_wt[parity][w2];
        if (w2 < wave) accp += v2;
        tsum += v2;
      }
      accp += lex;
      int c2 = INT_MAX, lp = -1;
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        accp += rv[j];
        if (!take_last && c2 == INT_MAX && accp > t) c2 = e + j;
        if (rv[j] > 0.0) lp = e + j;
      }
      c2 = wave_min_int_dpp(c2);
      lp = wave_max_int_dpp(lp);
      if (lane == 0) {
        if (c2 != INT_MAX) atomicMin(&s_cand, c2);
        if (lp >= 0) atomicMax(&s_last, lp);
      }
      run = tsum;
      __syncthreads();
      if (s_cand != INT_MAX) break;
    }
    tok = s_cand != INT_MAX ? s_cand : (s_last >= 0 ? s_last : V - 1);
  }
  if (threadIdx.x == 0) tokens[row] = tok;
}

// Greedy: the argmax of row g is computed only when every draft was accepted.
template <typename T, bool ALIGNED, bool RAGGED, bool ACCEPT>
__global__ __launch_bounds__(kSeqThreads) void k_greedy_seq(Args a) {
  __shared__ int s_tok[kMaxGamma];
  __shared__ float s_v[kSeqWaves];
  __shared__ int s_i[kSeqWaves];
  __shared__ int s_n;
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int base, g;
  if (!seq_geom<RAGGED>(a, b, base, g)) {
    if (threadIdx.x == 0) {
      atomicOr(a.err, SV_DATA_CU_GAMMA);
      a.acc[b] = -1;
    }
    return;
  }
  const int n = first_rejection<T, ACCEPT, true>(a, b, base, g, nullptr, s_tok, &s_n);
  for (int i = threadIdx.x; i < n; i += kSeqThreads) a.emitted[base + b + i] = a.ids[base + i];
  int tok = n < g ? s_tok[n] : -1;
  if (n == g) {  // the bonus row is read only when every draft was accepted
    const T* row = static_cast<const T*>(a.logits) + static_cast<size_t>(base + b + g) * a.V;
    float bv = -INFINITY;
    float nw = -INFINITY;  // NaN watch of the bonus row
    int bi = INT_MAX;
    if (ALIGNED) {
      const int g1 = a.V >> 3;
      int gi = threadIdx.x;
      if (gi < g1) bi = gi * kGroup;
      for (; gi + (kUnroll - 1) * kSeqThreads < g1; gi += kUnroll * kSeqThreads) {
        float xv[kUnroll][kGroup];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) load_group(row, static_cast<size_t>(gi + u * kSeqThreads) * kGroup, xv[u]);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          nw = nan_watch(nw, xv[u]);
#pragma unroll
          for (int j = 0; j < kGroup; ++j)
            if (xv[u][j] > bv) {
              bv = xv[u][j];
              bi = (gi + u * kSeqThreads) * kGroup + j;
            }
        }
      }
      for (; gi < g1; gi += kSeqThreads) {
        float xv[kGroup];
        load_group(row, static_cast<size_t>(gi) * kGroup, xv);
        nw = nan_watch(nw, xv);
#pragma unroll
        for (int j = 0; j < kGroup; ++j)
          if (xv[j] > bv) {
            bv = xv[j];
            bi = gi * kGroup + j;
          }
      }
    } else {
      int e = threadIdx.x;
      if (e < a.V) bi = e;
      for (; e < a.V; e += kSeqThreads) {
        const float xv = load_one(row, e);
        nw = nan_watch1(nw, xv);
        if (xv > bv) {
          bv = xv;
          bi = e;
        }
      }
    }
    flag_nan(nw, a.err, SV_DATA_NONFINITE);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float v2 = __shfl_xor(bv, o);
      const int i2 = __shfl_xor(bi, o);
      argmax_merge(bv, bi, v2, i2);
    }
    if (lane == 0) {
      s_v[wave] = bv;
      s_i[wave] = bi;
    }
    __syncthreads();
    float V = s_v[0];
    int I = s_i[0];
    for (int w = 1; w < kSeqWaves; ++w) argmax_merge(V, I, s_v[w], s_i[w]);
    tok = I;
  }
  if (threadIdx.x == 0) {
    a.acc[b] = n;
    a.emitted[base + b + n] = tok;
    a.rsum[b] = 0.f;
  }
  for (int i = n + 1 + threadIdx.x; i <= g; i += kSeqThreads) a.emitted[base + b + i] = -1;
}

// ============================================================== host side
constexpr int kKernels = 3;  // most kernels one call launches
constexpr int kEventsPerRun = 2 * kKernels;

// The launch sequences a call can take.
enum Path {
  kPathSample2 = 0, kPathGreedy2 = 1, kPathSample1 = 2, kPathGreedy1 = 3, kPathSample3 = 4, kPathRows = 5,
  kPathSample1R = 6, kPathGreedy1R = 7, kPathGreedyH = 8, kPathGreedyHR = 9, kPathGroup = 10, kPathTiny = 11,
  kPaths = 12
};
struct PathInfo {
  int nk;
  const char* names[kKernels];
};
const PathInfo kPathInfo[kPaths] = {
    {2, {"k_rowstats", "k_sample_seq"}},
    {2, {"k_rowargmax", "k_greedy_seq"}},
    {1, {"k_verify_seq", nullptr}},
    {1, {"k_greedy_seq1", nullptr}},
    {2, {"k_rowstats", "k_draw_part"}},
    {1, {"k_sample_rows", nullptr}},
    {2, {"k_order_by_gamma", "k_verify_seq"}},
    {2, {"k_order_by_gamma", "k_greedy_seq1"}},
    {1, {"k_greedy_help", nullptr}},
    {2, {"k_order_by_gamma", "k_greedy_help"}},
    {1, {"k_verify_group", nullptr}},
    {1, {"k_verify_tiny", nullptr}},
};

}  // namespace

struct spec_verify_ctx {
  int device = 0, V = 0, dtype = 0, max_batch = 0, max_rows = 0, max_gamma = 0, cus = 0;
  void* ws = nullptr;
  RowStat* p1 = nullptr;
  size_t p1_cap = 0;         // entries of p1
  bool no_helpers = false;   // greedy runs never take the helper plan (its counters carry host epochs)
  bool no_tagged = false;    // nor the small-batch plan's workgroups, whose records carry a host call tag
  int32_t* accept = nullptr;
  float2* lxq = nullptr;     // split rows: the draft's logit and q entry
  int32_t* s_acc = nullptr;  // sampling: accepted counts (all 0) of the verify launch
  float* s_rsum = nullptr;   // sampling: residual sums (all 0)
  int* err = nullptr;
  hipStream_t last_stream = nullptr;
  bool ran = false;
  // measurement: a start and a stop event per kernel and recorded run, for up to timing_cap runs
  int timing_cap = 0, timing_runs = 0;
  int timing_stride = 1;          // record one run in every timing_stride
  long long timing_seen = 0;      // runs seen since recording was armed
  hipEvent_t* ev = nullptr;
  int timing_path = -1;  // the path of the recorded runs (runs on another path are not recorded)
  int path_mode = SV_PATH_AUTO, last_path = SV_PATH_AUTO;
  // split draw of the two-launch plan (up to split_cap sequences)
  double* dsum = nullptr;
  int* dcnt = nullptr;
  int split_cap = 0;
  int* order = nullptr;  // [max_batch] sequence order of the one-launch plan (ragged batches)
  // greedy rows with helpers: per-sequence claim counter, participants and published minimum
  unsigned long long* gclaim = nullptr;
  unsigned long long* gpart = nullptr;
  unsigned long long* gbest = nullptr;
  unsigned int gepoch = 0;  // the last call's epoch (0 is never used: the arrays start at 0)
  // small-batch one-launch plan (up to grp_cap sequences)
  unsigned long long* pchunk = nullptr;
  unsigned long long* psum = nullptr;
  int grp_cap = 0;
  int grp_slots = 0;     // workgroups of k_verify_group resident at once (0: not yet known)
  unsigned ptag = 0;     // the last call's tag
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

// With timing on, each kernel is launched through hipExtLaunchKernel with a start and
// a stop event, which take the dispatch's own begin / end timestamps (the launch gap
// between kernels is not counted).
// Events of this run when it is recorded, else nullptr.
hipEvent_t* timing_slot(spec_verify_ctx* ctx, int path) {
  if (ctx->timing_runs >= ctx->timing_cap) return nullptr;
  if (ctx->timing_seen++ % ctx->timing_stride != 0) return nullptr;
  if (ctx->timing_runs > 0 && ctx->timing_path != path) return nullptr;
  ctx->timing_path = path;
  return ctx->ev + static_cast<size_t>(ctx->timing_runs) * kEventsPerRun;
}

hipError_t launch_one(const void* fn, dim3 grid, dim3 block, const Args& a, hipStream_t st, hipEvent_t* ev,
                      int k) {
  void* args[] = {const_cast<Args*>(&a)};
  return hipExtLaunchKernel(fn, grid, block, args, 0, st, ev ? ev[2 * k] : nullptr, ev ? ev[2 * k + 1] : nullptr,
                            0);
}

template <typename T, bool RG>
hipError_t launch_fused(spec_verify_ctx* ctx, const Args& a, hipStream_t st) {
  if (!RG && a.gamma == 0 && a.B > ctx->cus) {  // draws only: one workgroup per compute unit
    hipEvent_t* ev = timing_slot(ctx, kPathRows);
    const hipError_t e = launch_one(reinterpret_cast<const void*>(&k_sample_rows<T>), dim3(ctx->cus),
                                    dim3(kSeqThreads), a, st, ev, 0);
    if (e != hipSuccess) return e;
    if (ev) ++ctx->timing_runs;
    return hipGetLastError();
  }
  // a ragged batch with more sequences than compute units: longest draft first
  const bool ordered = RG && a.B > ctx->cus;
  Args ao = a;
  ao.order = ordered ? ctx->order : nullptr;
  hipEvent_t* ev = timing_slot(ctx, ordered ? kPathSample1R : kPathSample1);
  int k = 0;
  if (ordered) {
    const hipError_t e = launch_one(reinterpret_cast<const void*>(&k_order_by_gamma), dim3(1),
                                    dim3(kOrderThreads), ao, st, ev, k++);
    if (e != hipSuccess) return e;
  }
  const void* fn = reinterpret_cast<const void*>(&k_verify_seq<T, RG>);
  const hipError_t e = launch_one(fn, dim3(a.B), dim3(kSeqThreads), ao, st, ev, k);
  if (e != hipSuccess) return e;
  if (ev) ++ctx->timing_runs;
  return hipGetLastError();
}

template <typename T, bool RG>
hipError_t launch_fused_greedy(spec_verify_ctx* ctx, const Args& a, hipStream_t st) {
  const bool ordered = RG && a.B > ctx->cus;  // longest draft first, as for sampling
  Args ao = a;
  ao.order = ordered ? ctx->order : nullptr;
  // helpers while the batch is at most four times the compute units (the longest
  // sequences then set the time)
  const bool help = SV_GREEDY_HELP && !ctx->no_helpers && a.B >= ctx->cus && a.B <= 4 * ctx->cus;
  if (help) {
    ao.gclaim = ctx->gclaim;
    ao.gpart = ctx->gpart;
    ao.gbest = ctx->gbest;
    if (++ctx->gepoch == 0) ctx->gepoch = 1;
    ao.gepoch = ctx->gepoch;
    hipEvent_t* ev = timing_slot(ctx, ordered ? kPathGreedyHR : kPathGreedyH);
    int k = 0;
    if (ordered) {
      const hipError_t e = launch_one(reinterpret_cast<const void*>(&k_order_by_gamma), dim3(1),
                                      dim3(kOrderThreads), ao, st, ev, k++);
      if (e != hipSuccess) return e;
    }
    const hipError_t e = launch_one(reinterpret_cast<const void*>(&k_greedy_help<T, RG>),
                                    dim3(SV_GREEDY_WAVES * static_cast<unsigned>(a.B)), dim3(kSeqThreads), ao, st,
                                    ev, k);
    if (e != hipSuccess) return e;
    if (ev) ++ctx->timing_runs;
    return hipGetLastError();
  }
  hipEvent_t* ev = timing_slot(ctx, ordered ? kPathGreedy1R : kPathGreedy1);
  int k = 0;
  if (ordered) {
    const hipError_t e = launch_one(reinterpret_cast<const void*>(&k_order_by_gamma), dim3(1),
                                    dim3(kOrderThreads), ao, st, ev, k++);
    if (e != hipSuccess) return e;
  }
  // nontemporal row loads when every sequence has its own compute unit (measured with
  // inputs rotated past the last-level cache, gamma = 8, V = 152064 bf16: B = 255, 103.4
  // against 106.0 us with ordinary loads; B = 224, 101.5 against 103.5 us)
  const void* fn = a.B <= ctx->cus ? reinterpret_cast<const void*>(&k_greedy_seq1<T, RG, true>)
                                   : reinterpret_cast<const void*>(&k_greedy_seq1<T, RG, false>);
  const hipError_t e = launch_one(fn, dim3(a.B), dim3(kSeqThreads), ao, st, ev, k);
  if (e != hipSuccess) return e;
  if (ev) ++ctx->timing_runs;
  return hipGetLastError();
}

// Workgroups of k_verify_group resident on the device at once.
template <typename T>
int group_slots(int cus) {
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(&k_verify_group<T>),
                                                   kGrpThreads, 0) != hipSuccess || occ < 1)
    occ = 1;
  return cus * occ;
}

// The small-batch plan's geometry: chunks per draft row (split) and their width (span),
// so that all B x gamma x split workgroups are resident at once, at most kGrpMaxW per
// sequence; the drawn row's unit width and count. Rows of at most kTinyMaxV entries take
// one workgroup per sequence (k_verify_tiny, any B; *tiny set). False when the rows alone
// are more workgroups than that, or the workspace does not hold the batch.
bool group_grid(spec_verify_ctx* ctx, Args& a, int& grid, bool* tiny) {
  *tiny = false;
  if (a.gamma < 0 || a.gamma > kGrpMaxW) return false;
  if (a.V <= kTinyMaxV) {
    *tiny = true;
    grid = a.B;
    a.split = 1;
    a.span = a.V;
    const int per = (a.V + kGrpWaves - 1) / kGrpWaves;  // one unit per wave
    a.uw = (per + kGroup - 1) / kGroup * kGroup;
    a.nunits = (a.V + a.uw - 1) / a.uw;
    return true;
  }
  if (!ctx->pchunk || a.B > ctx->grp_cap) return false;
  if (ctx->grp_slots == 0)
    ctx->grp_slots = ctx->dtype == SV_BF16 ? group_slots<uint16_t>(ctx->cus) : group_slots<float>(ctx->cus);
  const int cap = min(ctx->grp_slots, kGrpMaxItems);
  int W;
  if (a.gamma == 0) {
    a.split = 1;
    a.span = a.V;
    W = 1;
  } else {
    const long long R = static_cast<long long>(a.B) * a.gamma;
    if (R > cap) return false;
    int s = static_cast<int>(min(static_cast<long long>(kMaxSplit), cap / R));
    s = min(s, kGrpMaxW / a.gamma);
    s = max(1, min(s, a.V / SV_SPLIT_MIN_SPAN));
    int span = (a.V + s - 1) / s;
    span = (span + kGroup - 1) / kGroup * kGroup;
    a.span = span;
    a.split = (a.V + span - 1) / span;
    W = a.gamma * a.split;
  }
  if (static_cast<long long>(a.B) * W > cap) return false;
  grid = a.B * W;
  // units of the drawn row: at most one per wave of the sequence's workgroups and 64 in
  // all, whole sweep iterations (a unit's loads are then issued together, without a
  // masked tail)
  const int units = min(kGrpMaxUnits, W * kGrpWaves);
  const int per = (a.V + units - 1) / units;
  a.uw = (per + kIter - 1) / kIter * kIter;
  a.nunits = (a.V + a.uw - 1) / a.uw;
  return true;
}

template <typename T>
hipError_t launch_group(spec_verify_ctx* ctx, const Args& a0, hipStream_t st, int grid, bool tiny) {
  hipEvent_t* ev = timing_slot(ctx, tiny ? kPathTiny : kPathGroup);
  Args a = a0;
  a.pchunk = ctx->pchunk;
  a.psum = ctx->psum;
  if (!tiny && ++ctx->ptag == 0) ctx->ptag = 1;
  a.ptag = ctx->ptag;
  const void* fn = tiny ? reinterpret_cast<const void*>(&k_verify_tiny<T>)
                        : reinterpret_cast<const void*>(&k_verify_group<T>);
  const hipError_t e = launch_one(fn, dim3(grid), dim3(kGrpThreads), a, st, ev, 0);
  if (e != hipSuccess) return e;
  if (ev) ++ctx->timing_runs;
  return hipGetLastError();
}

template <typename T, bool AL, bool RG, bool AC>
hipError_t launch_path(spec_verify_ctx* ctx, const Args& a, hipStream_t st, bool greedy) {
  hipEvent_t* ev = timing_slot(ctx, greedy ? kPathGreedy2 : kPathSample2);
  const bool rec = ev != nullptr;
  auto go = [&](const void* fn, dim3 grid, dim3 block, int k) -> hipError_t {
    return launch_one(fn, grid, block, a, st, ev, k);
  };
  hipError_t e = hipSuccess;
  if (a.R > 0) {
    const dim3 grid(static_cast<unsigned>(a.R) * a.split);
    e = greedy ? go(reinterpret_cast<const void*>(&k_rowargmax<T, AL, RG, AC>), grid, dim3(kThreads), 0)
               : go(reinterpret_cast<const void*>(&k_rowstats<T, AL, RG, AC>), grid, dim3(kThreads), 0);
  } else if (ev) {
    (void)hipEventRecord(ev[0], st);
    (void)hipEventRecord(ev[1], st);
  }
  if (e != hipSuccess) return e;
  e = greedy ? go(reinterpret_cast<const void*>(&k_greedy_seq<T, AL, RG, AC>), dim3(a.B), dim3(kSeqThreads), 1)
             : go(reinterpret_cast<const void*>(&k_sample_seq<T, AL, RG, AC>), dim3(a.B), dim3(kSeqThreads), 1);
  if (e != hipSuccess) return e;
  if (rec) ++ctx->timing_runs;
  return hipGetLastError();
}

// The split draw: with at most half as many sequences as compute units, two or four
// workgroups share the sweep of each drawn row (bf16 rows through the value table, fp32
// rows with exp2_tab): four when there are at least four compute units per sequence,
// else two. bf16 rows split only when the temperature admits the value table.
// Fewer slices when the row is too short for the last one to get any of it.
int split_slices(const spec_verify_ctx* ctx, const Args& a) {
  const bool bf16 = ctx->dtype == SV_BF16;
  if ((bf16 && a.tlo > a.thi) || a.B < 1 || a.B > ctx->split_cap) return 1;
  const int per = ctx->cus / a.B;
  int s = per >= kMaxSlices ? kMaxSlices : per >= 2 ? 2 : 1;
  while (s > 1) {
    const int ns = kSeqWaves * s;
    const long long w = bf16 ? sub_width(a.V, ns) : iter_width(a.V, ns);
    if (static_cast<long long>(ns - kSeqWaves) * w < a.V) break;
    s /= 2;
  }
  return s;
}

template <typename T, bool RG, bool AC>
hipError_t launch_split(spec_verify_ctx* ctx, const Args& a0, hipStream_t st, int nslice) {
  hipEvent_t* ev = timing_slot(ctx, kPathSample3);
  Args a = a0;
  a.nslice = nslice;
  a.dsum = ctx->dsum;
  a.dcnt = ctx->dcnt;
  hipError_t e = hipSuccess;
  if (a.R > 0) {
    e = launch_one(reinterpret_cast<const void*>(&k_rowstats<T, true, RG, AC>),
                   dim3(static_cast<unsigned>(a.R) * a.split), dim3(kThreads), a, st, ev, 0);
  } else if (ev) {
    (void)hipEventRecord(ev[0], st);
    (void)hipEventRecord(ev[1], st);
  }
  if (e != hipSuccess) return e;
  e = launch_one(reinterpret_cast<const void*>(&k_draw_part<T, RG, AC>), dim3(static_cast<unsigned>(a.B) * nslice),
                 dim3(kSeqThreads), a, st, ev, 1);
  if (e != hipSuccess) return e;
  if (ev) ++ctx->timing_runs;
  return hipGetLastError();
}

template <typename T, bool AL, bool RG>
hipError_t launch_ac(spec_verify_ctx* ctx, const Args& a, hipStream_t st, bool greedy) {
  if constexpr (AL) {
    const int ns = greedy ? 1 : split_slices(ctx, a);
    if (ns > 1)
      return a.split == 1 ? launch_split<T, RG, true>(ctx, a, st, ns) : launch_split<T, RG, false>(ctx, a, st, ns);
  }
  // rows that are not split run their accept test inside the row-statistics kernel
  return a.split == 1 ? launch_path<T, AL, RG, true>(ctx, a, st, greedy)
                      : launch_path<T, AL, RG, false>(ctx, a, st, greedy);
}

template <typename T>
hipError_t launch_dt(spec_verify_ctx* ctx, const Args& a, hipStream_t st, bool greedy, bool aligned, bool ragged) {
  if (aligned)
    return ragged ? launch_ac<T, true, true>(ctx, a, st, greedy) : launch_ac<T, true, false>(ctx, a, st, greedy);
  return ragged ? launch_ac<T, false, true>(ctx, a, st, greedy) : launch_ac<T, false, false>(ctx, a, st, greedy);
}

void free_events(spec_verify_ctx* ctx) {
  if (ctx->ev) {
    const size_t n = static_cast<size_t>(ctx->timing_cap) * kEventsPerRun;
    for (size_t i = 0; i < n; ++i)
      if (ctx->ev[i]) (void)hipEventDestroy(ctx->ev[i]);
    delete[] ctx->ev;
  }
  ctx->ev = nullptr;
  ctx->timing_cap = ctx->timing_runs = 0;
  ctx->timing_path = -1;
}

// Row-stats split: aim for >= SV_SPLIT_TARGET workgroups with >= SV_SPLIT_MIN_SPAN
// entries per split.
void choose_split(int R, int V, int& split, int& span) {
  int s = R > 0 ? (SV_SPLIT_TARGET + R - 1) / R : 1;
  s = s < 1 ? 1 : (s > kMaxSplit ? kMaxSplit : s);
  const int by_len = (V + SV_SPLIT_MIN_SPAN - 1) / SV_SPLIT_MIN_SPAN;
  if (s > by_len) s = by_len < 1 ? 1 : by_len;
  int sp = (V + s - 1) / s;
  sp = (sp + kGroup - 1) / kGroup * kGroup;
  split = (V + sp - 1) / sp;
  span = sp;
}

}  // namespace

namespace {
int run_impl(spec_verify_ctx* ctx, void* hip_stream, int batch, int gamma, const int32_t* cu_gamma,
             int total_draft_rows, float temperature, const void* logits, const float* q, bool onehot,
             const int32_t* draft_ids, const float* uniforms, int32_t* accepted_count, int32_t* emitted_tokens,
             float* residual_sum, float* p_draft) {
  if (!ctx) return SV_EINVAL;
  const int rc = spec_verify_check_args(
      ctx->V, ctx->dtype, ctx->max_batch, ctx->max_rows, ctx->max_gamma, batch, gamma, cu_gamma != nullptr,
      total_draft_rows, temperature, logits != nullptr, onehot || q != nullptr, draft_ids != nullptr,
      uniforms != nullptr, accepted_count != nullptr, emitted_tokens != nullptr, residual_sum != nullptr, ctx->msg,
      sizeof(ctx->msg));
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
  a.q = greedy || onehot ? nullptr : q;
  a.onehot = onehot && !greedy ? 1 : 0;
  a.nodraft = onehot ? 1 : 0;
  a.ids = draft_ids;
  a.u = greedy ? nullptr : uniforms;
  a.cu = cu_gamma;
  a.acc = accepted_count;
  a.emitted = emitted_tokens;
  a.rsum = residual_sum;
  a.pdraft = greedy ? nullptr : p_draft;
  a.p1 = ctx->p1;
  a.accept = ctx->accept;
  a.lxq = ctx->lxq;
  a.err = ctx->err;
  a.B = batch;
  a.gamma = cu_gamma ? -1 : gamma;
  a.V = ctx->V;
  a.R = total_draft_rows;
  a.max_gamma = ctx->max_gamma;
  choose_split(a.R, a.V, a.split, a.span);
  if (static_cast<size_t>(a.R) * a.split > ctx->p1_cap) {  // cannot happen within the max_* sizes
    set_msg(ctx->msg, sizeof(ctx->msg), "row statistics exceed the workspace");
    return SV_EINVAL;
  }
  const unsigned long long max_threads = 1ull << 32;
  if (static_cast<unsigned long long>(a.R) * a.split * kThreads >= max_threads ||
      static_cast<unsigned long long>(a.B) * kSeqThreads >= max_threads) {
    set_msg(ctx->msg, sizeof(ctx->msg), "launch grid too large: reduce the batch");
    return SV_EINVAL;
  }
  a.tlo = 1;
  a.thi = 0;  // no value table
  if (greedy) {
    a.k2 = 0.f;
    a.k2d = 0.0;
    a.kr = 1.0;
  } else {
    a.k2d = 1.4426950408889634 / static_cast<double>(temperature);
    a.k2 = static_cast<float>(a.k2d);
    a.kr = a.k2d / static_cast<double>(a.k2);
    // bf16 value table window: magnitudes below 2^etop, |x k2| < 990, kTabBinades octaves
    const int etop = static_cast<int>(floor(log2(990.0 / a.k2d)));
    const int be_hi = etop + 127 > 255 ? 255 : etop + 127;  // biased exponent, exclusive
    const int be_lo = be_hi - kTabBinades < 0 ? 0 : be_hi - kTabBinades;
    if (ctx->dtype == SV_BF16 && be_hi > be_lo) {
      a.tlo = be_lo * 128;
      a.thi = be_hi * 128 - 1;
    }
  }
  DeviceGuard guard(ctx->device);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const int gmax = cu_gamma ? ctx->max_gamma : gamma;
  const bool rg = cu_gamma != nullptr;
  // small batches of sampling rows, uniform gamma: one launch with the rows read in
  // parallel and the draws pooled (AUTO below the compute-unit count, or when asked)
  Args ga = a;
  int ggrid = 0;
  bool tiny = false;
  const bool grp_ok = !greedy && !rg && aligned && group_grid(ctx, ga, ggrid, &tiny) && (tiny || !ctx->no_tagged);
  // AUTO: short rows, or fewer sequences than compute units with fp32 logits (bf16 rows
  // drawn through the value table measured faster in two launches: C3 rows at B = 32 and
  // 64, 26.5 and 32.7 us against 29.5 and 34.2 us)
  const bool table = ctx->dtype == SV_BF16 && a.tlo <= a.thi;
  const bool pooled = grp_ok && (ctx->path_mode == SV_PATH_POOLED ||
                                 (ctx->path_mode == SV_PATH_AUTO && (tiny || (batch < ctx->cus && !table))));
  // AUTO takes one launch from a fraction of the compute-unit count on: below it the two
  // launches spread the rows over every compute unit and finish first, above it one
  // workgroup per sequence does. Measured on MI355X with inputs rotated past the
  // last-level cache (us per call, one / two launches): sampling, gamma = 4, V = 128256
  // bf16: B = 128 57.7 / 51.3, B = 144 58.8 / 59.8, B = 192 62.4 / 68.7; greedy,
  // gamma = 8, V = 152064 bf16: B = 192 100.7 / 95.8, B = 208 101.4 / 103.2.
  const int one_min = greedy ? (4 * ctx->cus + 4) / 5 : (11 * ctx->cus + 19) / 20;
  const bool fused = !pooled && ctx->path_mode != SV_PATH_TWO_LAUNCH && ctx->path_mode != SV_PATH_POOLED && aligned &&
                     gmax <= kFuseMaxGamma && (ctx->path_mode == SV_PATH_ONE_LAUNCH || batch >= one_min);
  hipError_t e;
  if (pooled)
    e = ctx->dtype == SV_BF16 ? launch_group<uint16_t>(ctx, ga, st, ggrid, tiny)
                              : launch_group<float>(ctx, ga, st, ggrid, tiny);
  else if (fused && greedy)
    e = ctx->dtype == SV_BF16
            ? (rg ? launch_fused_greedy<uint16_t, true>(ctx, a, st) : launch_fused_greedy<uint16_t, false>(ctx, a, st))
            : (rg ? launch_fused_greedy<float, true>(ctx, a, st) : launch_fused_greedy<float, false>(ctx, a, st));
  else if (fused)
    e = ctx->dtype == SV_BF16 ? (rg ? launch_fused<uint16_t, true>(ctx, a, st) : launch_fused<uint16_t, false>(ctx, a, st))
                              : (rg ? launch_fused<float, true>(ctx, a, st) : launch_fused<float, false>(ctx, a, st));
  else
    e = ctx->dtype == SV_BF16 ? launch_dt<uint16_t>(ctx, a, st, greedy, aligned, rg)
                              : launch_dt<float>(ctx, a, st, greedy, aligned, rg);
  if (e != hipSuccess) return hip_fail(ctx, "kernel launch", e);
  ctx->last_stream = st;
  ctx->ran = true;
  ctx->last_path = pooled ? SV_PATH_POOLED : fused ? SV_PATH_ONE_LAUNCH : SV_PATH_TWO_LAUNCH;
  return SV_OK;
}

// ---------------------------------------------------------------- vocabulary shards
hipError_t launch_vs(const void* fn, unsigned grid, unsigned block, const Args& a, const VShard& vs,
                     hipStream_t st) {
  void* args[] = {const_cast<Args*>(&a), const_cast<VShard*>(&vs)};
  return hipExtLaunchKernel(fn, dim3(grid), dim3(block), args, 0, st, nullptr, nullptr, 0);
}

// Checks shared by the three shard steps; fills a (a.V = this shard's width) and vs.
// has_* name the pointers the step needs (the others count as present).
int vshard_prepare(spec_verify_ctx* ctx, const spec_vshard* sh, int batch, int gamma, const int32_t* cu_gamma,
                   int total_draft_rows, float temperature, const void* logits, bool has_q, bool has_ids,
                   bool has_u, bool has_outputs, Args& a, VShard& vs) {
  if (!ctx) return SV_EINVAL;
  auto bad = [&](const char* m) {
    set_msg(ctx->msg, sizeof(ctx->msg), m);
    return SV_EINVAL;
  };
  if (!sh || !sh->bounds) return bad("the shard description or its bounds is NULL");
  const int G = sh->shards;
  if (G < 1 || G > kMaxShards) return bad("shards must be in [1, 64]");
  if (sh->shard < 0 || sh->shard >= G) return bad("shard must be in [0, shards)");
  if (sh->bounds[0] != 0 || sh->bounds[G] != sh->vocab_total) return bad("bounds must run from 0 to vocab_total");
  for (int k = 0; k < G; ++k)
    if (sh->bounds[k + 1] <= sh->bounds[k]) return bad("bounds must increase");
  if (sh->bounds[sh->shard + 1] - sh->bounds[sh->shard] != ctx->V)
    return bad("the context's vocab must equal this shard's width");
  const int rc = spec_verify_check_args(ctx->V, ctx->dtype, ctx->max_batch, ctx->max_rows, ctx->max_gamma, batch,
                                        gamma, cu_gamma != nullptr, total_draft_rows, temperature, logits != nullptr,
                                        has_q, has_ids, has_u, has_outputs, has_outputs, has_outputs, ctx->msg,
                                        sizeof(ctx->msg));
  if (rc != SV_OK) return rc;
  if (cu_gamma && batch > kMaxRaggedBatch) return bad("ragged batches (cu_gamma) are limited to 65536 sequences");
  const bool greedy = temperature == 0.f;
  a = Args{};
  a.logits = logits;
  a.cu = cu_gamma;
  a.err = ctx->err;
  a.B = batch;
  a.gamma = cu_gamma ? -1 : gamma;
  a.V = ctx->V;
  a.R = total_draft_rows;
  a.max_gamma = ctx->max_gamma;
  a.tlo = 1;
  a.thi = 0;
  a.k2d = greedy ? 0.0 : 1.4426950408889634 / static_cast<double>(temperature);
  a.k2 = static_cast<float>(a.k2d);
  a.kr = greedy ? 1.0 : a.k2d / static_cast<double>(a.k2);
  vs = VShard{};
  vs.G = G;
  vs.me = sh->shard;
  vs.nrec = total_draft_rows + (greedy ? batch : 0);
  for (int k = 0; k <= G; ++k) vs.vb[k] = sh->bounds[k];
  if (static_cast<unsigned long long>(vs.nrec) * kThreads >= (1ull << 32)) return bad("launch grid too large");
  return SV_OK;
}

bool vshard_aligned(const spec_verify_ctx* ctx, const void* logits, const float* q, bool greedy) {
  return ctx->V % kGroup == 0 && reinterpret_cast<uintptr_t>(logits) % 16 == 0 &&
         (greedy || reinterpret_cast<uintptr_t>(q) % 16 == 0);
}

// One template instance per (dtype, aligned, ragged, greedy).
template <template <typename, bool, bool, bool> class K>
const void* vs_pick(bool bf16, bool al, bool rg, bool gr) {
#define SV_VS_K(T, A, R, G) reinterpret_cast<const void*>(K<T, A, R, G>::fn)
  if (bf16) {
    if (al) return rg ? (gr ? SV_VS_K(uint16_t, true, true, true) : SV_VS_K(uint16_t, true, true, false))
                      : (gr ? SV_VS_K(uint16_t, true, false, true) : SV_VS_K(uint16_t, true, false, false));
    return rg ? (gr ? SV_VS_K(uint16_t, false, true, true) : SV_VS_K(uint16_t, false, true, false))
              : (gr ? SV_VS_K(uint16_t, false, false, true) : SV_VS_K(uint16_t, false, false, false));
  }
  if (al) return rg ? (gr ? SV_VS_K(float, true, true, true) : SV_VS_K(float, true, true, false))
                    : (gr ? SV_VS_K(float, true, false, true) : SV_VS_K(float, true, false, false));
  return rg ? (gr ? SV_VS_K(float, false, true, true) : SV_VS_K(float, false, true, false))
            : (gr ? SV_VS_K(float, false, false, true) : SV_VS_K(float, false, false, false));
#undef SV_VS_K
}
template <typename T, bool A, bool R, bool G> struct VsRows { static constexpr auto fn = &k_vs_rows<T, A, R, G>; };
template <typename T, bool A, bool R, bool G> struct VsDecide { static constexpr auto fn = &k_vs_decide<T, A, R, G>; };
template <typename T, bool A, bool R, bool G> struct VsFinish { static constexpr auto fn = &k_vs_finish<T, A, R>; };

// ---------------------------------------------------------------- workspace layout
// Byte offsets of a context's device arrays in one block, each 256-byte aligned: the
// row statistics (p1_cap entries), per draft row the decision and the draft's logit and
// q entry, per sequence the sampling-mode scratch outputs, the ordering and the three
// greedy-helper counters, the split draw's sums and counts (split_cap sequences), and
// the error word.
struct WsLayout {
  size_t p1, accept, lxq, s_acc, s_rsum, order, gclaim, gpart, gbest, dsum, dcnt, err;
  size_t pchunk, psum, total;
  size_t p1_cap;
  int split_cap, grp_cap;
};
constexpr size_t ws_up(size_t x) { return (x + 255) / 256 * 256; }
constexpr WsLayout ws_layout(size_t p1_cap, int max_rows, int max_batch, int split_cap, int grp_cap) {
  const size_t rows = static_cast<size_t>(max_rows > 0 ? max_rows : 1);
  const size_t seqs = static_cast<size_t>(max_batch > 0 ? max_batch : 1);
  const size_t cap = static_cast<size_t>(split_cap > 0 ? split_cap : 0);
  WsLayout L{};
  size_t o = 0;
  L.p1 = o;      o += ws_up(sizeof(RowStat) * (p1_cap > 0 ? p1_cap : 1));
  L.accept = o;  o += ws_up(sizeof(int32_t) * rows);
  L.lxq = o;     o += ws_up(sizeof(float2) * rows);
  L.s_acc = o;   o += ws_up(sizeof(int32_t) * seqs);
  L.s_rsum = o;  o += ws_up(sizeof(float) * seqs);
  L.order = o;   o += ws_up(sizeof(int32_t) * seqs);
  L.gclaim = o;  o += ws_up(sizeof(unsigned long long) * seqs);
  L.gpart = o;   o += ws_up(sizeof(unsigned long long) * seqs);
  L.gbest = o;   o += ws_up(sizeof(unsigned long long) * seqs);
  L.dsum = o;    o += ws_up(sizeof(double) * 3 * kMaxSub * cap);
  L.dcnt = o;    o += ws_up(sizeof(int) * (cap > 0 ? cap : 1));
  L.err = o;     o += 256;
  const size_t gc = static_cast<size_t>(grp_cap > 0 ? grp_cap : 0);
  L.pchunk = o;  o += gc > 0 ? ws_up(sizeof(unsigned long long) * 4 * kGrpMaxItems) : 0;
  L.psum = o;    o += ws_up(sizeof(unsigned long long) * kSumWords * kGrpMaxUnits * gc);
  L.total = o;
  L.p1_cap = p1_cap;
  L.split_cap = split_cap;
  L.grp_cap = grp_cap;
  return L;
}
void ws_assign(spec_verify_ctx* ctx, const WsLayout& L, char* base) {
  ctx->p1 = reinterpret_cast<RowStat*>(base + L.p1);
  ctx->p1_cap = L.p1_cap;
  ctx->accept = reinterpret_cast<int32_t*>(base + L.accept);
  ctx->lxq = reinterpret_cast<float2*>(base + L.lxq);
  ctx->s_acc = reinterpret_cast<int32_t*>(base + L.s_acc);
  ctx->s_rsum = reinterpret_cast<float*>(base + L.s_rsum);
  ctx->order = reinterpret_cast<int*>(base + L.order);
  ctx->gclaim = reinterpret_cast<unsigned long long*>(base + L.gclaim);
  ctx->gpart = reinterpret_cast<unsigned long long*>(base + L.gpart);
  ctx->gbest = reinterpret_cast<unsigned long long*>(base + L.gbest);
  ctx->split_cap = L.split_cap;
  ctx->dsum = L.split_cap > 0 ? reinterpret_cast<double*>(base + L.dsum) : nullptr;
  ctx->dcnt = L.split_cap > 0 ? reinterpret_cast<int*>(base + L.dcnt) : nullptr;
  ctx->err = reinterpret_cast<int*>(base + L.err);
  ctx->grp_cap = L.grp_cap;
  ctx->pchunk = L.grp_cap > 0 ? reinterpret_cast<unsigned long long*>(base + L.pchunk) : nullptr;
  ctx->psum = L.grp_cap > 0 ? reinterpret_cast<unsigned long long*>(base + L.psum) : nullptr;
}

// The no-allocation entry point's workspace: a static device array of the layout above
// for at most kStaticMaxBatch sequences and kStaticMaxRows draft rows (row statistics
// for R x split <= R + SV_SPLIT_TARGET entries, the split draw for 128 sequences).
constexpr int kStaticMaxBatch = SV_STATIC_MAX_BATCH;
constexpr int kStaticMaxRows = SV_STATIC_MAX_ROWS;
constexpr int kStaticSplitCap = 128;
constexpr WsLayout kStaticLayout =
    ws_layout(kStaticMaxRows + SV_SPLIT_TARGET, kStaticMaxRows, kStaticMaxBatch, kStaticSplitCap, kStaticMaxBatch);
constexpr int kStaticMaxDevices = 64;
static_assert(kStaticLayout.total <= static_cast<size_t>(SV_STATIC_SCRATCH_MAX_BYTES), "static workspace size");
static_assert(SV_STATIC_MAX_GAMMA == kFuseMaxGamma, "the static entry point's gamma limit");

// Set-up of the static workspace: the split draw's counts to 0 and the small-batch
// plan's records and unit sums to tag 0, which no call uses.
__global__ void k_static_setup(char* ws) {
  int* dcnt = reinterpret_cast<int*>(ws + kStaticLayout.dcnt);
  for (int i = threadIdx.x; i < kStaticSplitCap; i += blockDim.x) dcnt[i] = 0;
  unsigned long long* tail = reinterpret_cast<unsigned long long*>(ws + kStaticLayout.pchunk);
  const size_t words = (kStaticLayout.total - kStaticLayout.pchunk) / sizeof(unsigned long long);
  for (size_t i = threadIdx.x; i < words; i += blockDim.x) tail[i] = 0ull;
}

}  // namespace

// One copy per device, held until the process ends. In host code this name is a stand-in,
// not a device address: kernels get the address hipGetSymbolAddress returns for the device.
static __device__ __align__(256) unsigned char scratch[kStaticLayout.total];

namespace {
struct StaticDevice {
  char* ptr = nullptr;  // this device's copy of `scratch`
  int cus = 0;
  int grp_slots[2] = {0, 0};  // workgroups of k_verify_group resident at once: fp32, bf16 logits
};
StaticDevice g_static[kStaticMaxDevices];
std::mutex g_static_mu;
thread_local char g_static_msg[512];

// Once per device, with the device current: the address of its copy of `scratch` and its
// compute-unit count; the split draw's counts are cleared on `st` (a small kernel, so the
// set-up can also be captured into a graph). Returns SV_OK or SV_EHIP.
int static_device(int device, hipStream_t st, StaticDevice& out) {
  std::lock_guard<std::mutex> lock(g_static_mu);
  StaticDevice& d = g_static[device];
  if (!d.ptr) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      snprintf(g_static_msg, sizeof(g_static_msg), "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      return SV_EHIP;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) cus = 256;
    hipLaunchKernelGGL(k_static_setup, dim3(1), dim3(256), 0, st, static_cast<char*>(p));
    e = hipGetLastError();
    if (e != hipSuccess) {
      snprintf(g_static_msg, sizeof(g_static_msg), "kernel launch: %s", hipGetErrorString(e));
      return SV_EHIP;
    }
    d.grp_slots[0] = group_slots<float>(cus);
    d.grp_slots[1] = group_slots<uint16_t>(cus);
    d.cus = cus;
    d.ptr = static_cast<char*>(p);
  }
  out = d;
  return SV_OK;
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
  if (vocab < 1 || vocab > kMaxVocab || max_batch < 0 || max_draft_rows < 0 || max_gamma < 0 ||
      max_gamma > kMaxGamma ||
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
  if (hipDeviceGetAttribute(&ctx->cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) ctx->cus = 256;
  const int by_len = (vocab + SV_SPLIT_MIN_SPAN - 1) / SV_SPLIT_MIN_SPAN;
  const int max_split = by_len < kMaxSplit ? by_len : kMaxSplit;
  const WsLayout L = ws_layout(static_cast<size_t>(max_draft_rows > 0 ? max_draft_rows : 1) * max_split,
                               max_draft_rows, max_batch, max_batch < kSplitMaxB ? max_batch : kSplitMaxB,
                               max_batch < kGrpMaxItems ? max_batch : kGrpMaxItems);
  if (hipMalloc(&ctx->ws, L.total) != hipSuccess) {
    delete ctx;
    return SV_ENOMEM;
  }
  ws_assign(ctx, L, static_cast<char*>(ctx->ws));
  if (hipMemset(ctx->ws, 0, L.total) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
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
  return run_impl(ctx, hip_stream, batch, gamma, cu_gamma, total_draft_rows, temperature, logits, q, false,
                  draft_ids, uniforms, accepted_count, emitted_tokens, residual_sum, p_draft);
}

int spec_verify_run_static(int device, void* hip_stream, int vocab, int logits_dtype, int batch, int gamma,
                           const int32_t* cu_gamma, int total_draft_rows, float temperature, const void* logits,
                           const float* q, const int32_t* draft_ids, const float* uniforms,
                           int32_t* accepted_count, int32_t* emitted_tokens, float* residual_sum, float* p_draft,
                           int32_t* data_flags) {
  auto bad = [&](const char* m) {
    set_msg(g_static_msg, sizeof(g_static_msg), m);
    return SV_EINVAL;
  };
  if (vocab < 1 || vocab > kMaxVocab) return bad("vocab must be in [1, 2^24]");
  if (logits_dtype != SV_F32 && logits_dtype != SV_BF16) return bad("logits_dtype must be SV_F32 or SV_BF16");
  if (batch > kStaticMaxBatch) return bad("batch exceeds SV_STATIC_MAX_BATCH (1024) of the static workspace");
  if (total_draft_rows > kStaticMaxRows)
    return bad("total_draft_rows exceeds SV_STATIC_MAX_ROWS (16384) of the static workspace");
  if (batch > 0 && !data_flags) return bad("data_flags is NULL");
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev || device >= kStaticMaxDevices)
    return bad("no such device");
  if (batch <= 0) {  // checked like spec_verify_run; nothing to enqueue
    const int rc = spec_verify_check_args(vocab, logits_dtype, kStaticMaxBatch, kStaticMaxRows, kFuseMaxGamma,
                                          batch, gamma, cu_gamma != nullptr, total_draft_rows, temperature, 1, 1,
                                          1, 1, 1, 1, 1, g_static_msg, sizeof(g_static_msg));
    return rc;
  }
  DeviceGuard guard(device);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  StaticDevice dv;
  const int rc0 = static_device(device, st, dv);
  if (rc0 != SV_OK) return rc0;
  // a context on the stack that describes the static workspace: the same checks, plans
  // and kernels as spec_verify_run, minus the greedy helpers
  spec_verify_ctx c;
  c.device = device;
  c.V = vocab;
  c.dtype = logits_dtype;
  c.max_batch = kStaticMaxBatch;
  c.max_rows = kStaticMaxRows;
  c.max_gamma = SV_STATIC_MAX_GAMMA;
  c.cus = dv.cus;
  c.no_helpers = true;
  c.no_tagged = true;
  c.grp_slots = dv.grp_slots[logits_dtype == SV_BF16 ? 1 : 0];
  ws_assign(&c, kStaticLayout, dv.ptr);
  c.err = data_flags;
  const int rc = run_impl(&c, hip_stream, batch, gamma, cu_gamma, total_draft_rows, temperature, logits, q, false,
                          draft_ids, uniforms, accepted_count, emitted_tokens, residual_sum, p_draft);
  set_msg(g_static_msg, sizeof(g_static_msg), c.msg);
  return rc;
}

int spec_verify_run_onehot(spec_verify_ctx* ctx, void* hip_stream, int batch, int gamma, const int32_t* cu_gamma,
                           int total_draft_rows, float temperature, const void* logits, const int32_t* draft_ids,
                           const float* uniforms, int32_t* accepted_count, int32_t* emitted_tokens,
                           float* residual_sum, float* p_draft) {
  return run_impl(ctx, hip_stream, batch, gamma, cu_gamma, total_draft_rows, temperature, logits, nullptr, true,
                  draft_ids, uniforms, accepted_count, emitted_tokens, residual_sum, p_draft);
}


int spec_vshard_rows(spec_verify_ctx* ctx, void* hip_stream, const spec_vshard* sh, int batch, int gamma,
                     const int32_t* cu_gamma, int total_draft_rows, float temperature, const void* logits,
                     const float* q, const int32_t* draft_ids, void* rec) {
  Args a;
  VShard vs;
  const bool greedy = temperature == 0.f;
  int rc = vshard_prepare(ctx, sh, batch, gamma, cu_gamma, total_draft_rows, temperature, logits, q != nullptr,
                          draft_ids != nullptr, true, true, a, vs);
  if (rc != SV_OK) return rc;
  if (vs.nrec == 0) return SV_OK;
  if (!rec) {
    set_msg(ctx->msg, sizeof(ctx->msg), "rec is NULL");
    return SV_EINVAL;
  }
  a.q = greedy ? nullptr : q;
  a.ids = draft_ids;
  vs.rec = static_cast<ShardRec*>(rec);
  DeviceGuard guard(ctx->device);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const void* fn = vs_pick<VsRows>(ctx->dtype == SV_BF16, vshard_aligned(ctx, logits, q, greedy), cu_gamma != nullptr,
                                   greedy);
  const hipError_t e = launch_vs(fn, static_cast<unsigned>(vs.nrec), kThreads, a, vs, st);
  if (e != hipSuccess) return hip_fail(ctx, "kernel launch", e);
  ctx->last_stream = st;
  ctx->ran = true;
  return SV_OK;
}

int spec_vshard_decide(spec_verify_ctx* ctx, void* hip_stream, const spec_vshard* sh, int batch, int gamma,
                       const int32_t* cu_gamma, int total_draft_rows, float temperature, const void* logits,
                       const float* q, const int32_t* draft_ids, const float* uniforms, const void* rec_all,
                       int32_t* accepted_count, int32_t* emitted_tokens, float* residual_sum, float* p_draft,
                       double* part, double* local) {
  Args a;
  VShard vs;
  const bool greedy = temperature == 0.f;
  int rc = vshard_prepare(ctx, sh, batch, gamma, cu_gamma, total_draft_rows, temperature, logits, q != nullptr,
                          draft_ids != nullptr, uniforms != nullptr,
                          accepted_count && emitted_tokens && residual_sum, a, vs);
  if (rc != SV_OK) return rc;
  if (batch == 0) return SV_OK;
  if ((vs.nrec > 0 && !rec_all) || (!greedy && (!part || !local))) {
    set_msg(ctx->msg, sizeof(ctx->msg), "rec_all, part or local is NULL");
    return SV_EINVAL;
  }
  a.V = sh->vocab_total;  // ids are checked against the whole vocabulary
  a.q = greedy ? nullptr : q;
  a.ids = draft_ids;
  a.u = greedy ? nullptr : uniforms;
  a.acc = accepted_count;
  a.emitted = emitted_tokens;
  a.rsum = residual_sum;
  a.pdraft = greedy ? nullptr : p_draft;
  vs.all = static_cast<const ShardRec*>(rec_all);
  vs.part = part;
  vs.loc = local;
  DeviceGuard guard(ctx->device);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const void* fn = vs_pick<VsDecide>(ctx->dtype == SV_BF16, vshard_aligned(ctx, logits, q, greedy),
                                     cu_gamma != nullptr, greedy);
  const hipError_t e = launch_vs(fn, static_cast<unsigned>(batch), kSeqThreads, a, vs, st);
  if (e != hipSuccess) return hip_fail(ctx, "kernel launch", e);
  ctx->last_stream = st;
  ctx->ran = true;
  return SV_OK;
}

int spec_vshard_finish(spec_verify_ctx* ctx, void* hip_stream, const spec_vshard* sh, int batch, int gamma,
                       const int32_t* cu_gamma, int total_draft_rows, float temperature, const void* logits,
                       const float* q, const float* uniforms, const double* part_all, const double* local,
                       int32_t* emitted_tokens, float* residual_sum) {
  Args a;
  VShard vs;
  const bool greedy = temperature == 0.f;
  int rc = vshard_prepare(ctx, sh, batch, gamma, cu_gamma, total_draft_rows, temperature, logits, q != nullptr,
                          true, uniforms != nullptr, emitted_tokens && residual_sum, a, vs);
  if (rc != SV_OK) return rc;
  if (batch == 0 || greedy) return SV_OK;  // at T = 0 the decision step wrote every output
  if (!part_all || !local) {
    set_msg(ctx->msg, sizeof(ctx->msg), "part_all or local is NULL");
    return SV_EINVAL;
  }
  a.V = sh->vocab_total;
  a.q = q;
  a.u = uniforms;
  a.emitted = emitted_tokens;
  a.rsum = residual_sum;
  vs.part_all = part_all;
  vs.loc = const_cast<double*>(local);
  DeviceGuard guard(ctx->device);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const void* fn = vs_pick<VsFinish>(ctx->dtype == SV_BF16, vshard_aligned(ctx, logits, q, false),
                                     cu_gamma != nullptr, false);
  const hipError_t e = launch_vs(fn, static_cast<unsigned>(batch), kSeqThreads, a, vs, st);
  if (e != hipSuccess) return hip_fail(ctx, "kernel launch", e);
  ctx->last_stream = st;
  ctx->ran = true;
  return SV_OK;
}

int spec_sample_run(spec_verify_ctx* ctx, void* hip_stream, int rows, int mode, float temperature, const void* x,
                    const float* uniforms, int32_t* tokens) {
  if (!ctx) return SV_EINVAL;
  auto bad = [&](const char* m) {
    set_msg(ctx->msg, sizeof(ctx->msg), m);
    return SV_EINVAL;
  };
  if (rows < 0) return bad("rows must be >= 0");
  if (rows > ctx->max_batch) return bad("rows exceeds max_batch");
  if (mode != SV_SAMPLE_LOGITS && mode != SV_SAMPLE_WEIGHTS) return bad("mode must be SV_SAMPLE_LOGITS or SV_SAMPLE_WEIGHTS");
  if (mode == SV_SAMPLE_LOGITS && !(temperature >= 0.f && temperature <= FLT_MAX))
    return bad("temperature must be finite and >= 0");
  if (rows == 0) return SV_OK;
  if (!x || !tokens) return bad("x or tokens is NULL");
  const bool greedy = mode == SV_SAMPLE_LOGITS && temperature == 0.f;
  if (!greedy && !uniforms) return bad("uniforms is NULL");
  if (mode == SV_SAMPLE_LOGITS) {
    // the draw of a round with no drafts: row b is the target row, slot b its uniform
    const int rc = spec_verify_run(ctx, hip_stream, rows, 0, nullptr, 0, temperature, x, nullptr, nullptr,
                                   uniforms, ctx->s_acc, tokens, ctx->s_rsum, nullptr);
    return rc;
  }
  if (reinterpret_cast<uintptr_t>(x) % 4 != 0) return bad("weights not aligned to 4 bytes");
  const bool aligned = ctx->V % kGroup == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0;
  DeviceGuard guard(ctx->device);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const float* w = static_cast<const float*>(x);
  if (aligned)
    hipLaunchKernelGGL((k_sample_weights<true>), dim3(rows), dim3(kSeqThreads), 0, st, w, uniforms, tokens, ctx->err, ctx->V);
  else
    hipLaunchKernelGGL((k_sample_weights<false>), dim3(rows), dim3(kSeqThreads), 0, st, w, uniforms, tokens, ctx->err, ctx->V);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(ctx, "kernel launch", e);
  ctx->last_stream = st;
  ctx->ran = true;
  return SV_OK;
}

int spec_ngram_propose(spec_verify_ctx* ctx, void* hip_stream, int batch, const int32_t* tokens,
                       const int32_t* cu_ctx, int total_tokens, int n_min, int n_max, int gamma,
                       int32_t* draft_ids, int32_t* draft_len) {
  if (!ctx) return SV_EINVAL;
  auto bad = [&](const char* m) {
    set_msg(ctx->msg, sizeof(ctx->msg), m);
    return SV_EINVAL;
  };
  if (batch < 0) return bad("batch must be >= 0");
  if (total_tokens < 0) return bad("total_tokens must be >= 0");
  if (!(n_min >= 1 && n_min <= n_max && n_max <= SV_NGRAM_MAX_N))
    return bad("need 1 <= n_min <= n_max <= SV_NGRAM_MAX_N");
  if (gamma < 0 || gamma > 1024) return bad("gamma must be in [0, 1024]");
  if (batch == 0) return SV_OK;
  if (!cu_ctx || !draft_len) return bad("cu_ctx or draft_len is NULL");
  if (total_tokens > 0 && !tokens) return bad("tokens is NULL");
  if (gamma > 0 && !draft_ids) return bad("draft_ids is NULL");
  DeviceGuard guard(ctx->device);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  NgramArgs a{};
  a.tok = tokens;
  a.cu = cu_ctx;
  a.ids = draft_ids;
  a.len = draft_len;
  a.err = ctx->err;
  a.B = batch;
  a.total = total_tokens;
  a.n_min = n_min;
  a.n_max = n_max;
  a.gamma = gamma;
  const hipError_t e = sv_launch_ngram(a, st);
  if (e != hipSuccess) return hip_fail(ctx, "kernel launch", e);
  ctx->last_stream = st;
  ctx->ran = true;
  return SV_OK;
}

int spec_adapt_gamma(spec_verify_ctx* ctx, void* hip_stream, int batch, const int32_t* accepted_count,
                     int32_t* gamma, int32_t* streak, int gamma_max, int up_after, int down_after,
                     int32_t* cu_gamma_next) {
  if (!ctx) return SV_EINVAL;
  auto bad = [&](const char* m) {
    set_msg(ctx->msg, sizeof(ctx->msg), m);
    return SV_EINVAL;
  };
  if (batch < 0 || batch > kAdaptMaxBatch) return bad("batch must be in [0, 65536]");
  if (gamma_max < 1 || gamma_max > 1024) return bad("gamma_max must be in [1, 1024]");
  if (up_after < 1 || down_after < 1) return bad("up_after and down_after must be >= 1");
  if (batch == 0) return SV_OK;
  if (!accepted_count || !gamma || !streak || !cu_gamma_next) return bad("a state or output pointer is NULL");
  DeviceGuard guard(ctx->device);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  AdaptArgs a{};
  a.acc = accepted_count;
  a.gamma = gamma;
  a.streak = streak;
  a.cu = cu_gamma_next;
  a.err = ctx->err;
  a.B = batch;
  a.gmax = gamma_max;
  a.up = up_after;
  a.down = down_after;
  const hipError_t e = sv_launch_adapt(a, st);
  if (e != hipSuccess) return hip_fail(ctx, "kernel launch", e);
  ctx->last_stream = st;
  ctx->ran = true;
  return SV_OK;
}

int spec_verify_set_path(spec_verify_ctx* ctx, int mode) {
  if (!ctx || (mode != SV_PATH_AUTO && mode != SV_PATH_TWO_LAUNCH && mode != SV_PATH_ONE_LAUNCH &&
               mode != SV_PATH_POOLED))
    return SV_EINVAL;
  ctx->path_mode = mode;
  return SV_OK;
}

int spec_verify_last_path(const spec_verify_ctx* ctx) { return ctx ? ctx->last_path : -SV_EINVAL; }

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
  snprintf(ctx->msg, sizeof(ctx->msg), "device data error flags 0x%x:%s%s%s%s%s%s%s", flag,
           (flag & SV_DATA_DRAFT_ID) ? " draft-id-out-of-range" : "",
           (flag & SV_DATA_NONFINITE) ? " non-finite-normaliser" : "",
           (flag & SV_DATA_UNIFORM) ? " uniform-out-of-[0,1)" : "",
           (flag & SV_DATA_CU_GAMMA) ? " malformed-cu_gamma" : "",
           (flag & SV_DATA_CONTEXT) ? " malformed-cu_ctx" : "",
           (flag & SV_DATA_STATE) ? " adaptive-state-out-of-range" : "",
           (flag & SV_DATA_STALL) ? " internal-wait-bound-reached" : "");
  return SV_EDATA;
}

const char* spec_verify_last_error(const spec_verify_ctx* ctx) { return ctx ? ctx->msg : g_static_msg; }

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
  const size_t n = static_cast<size_t>(runs) * kEventsPerRun;
  ctx->ev = new (std::nothrow) hipEvent_t[n]();
  if (!ctx->ev) return SV_ENOMEM;
  ctx->timing_cap = runs;
  ctx->timing_seen = 0;
  // The events only carry timestamps, read after the stream has finished: recording them
  // needs no system-scope release (an L2 write-back between the kernels they bracket).
  for (size_t i = 0; i < n; ++i) {
    const hipError_t e = hipEventCreateWithFlags(&ctx->ev[i], hipEventDisableSystemFence);
    if (e != hipSuccess) {
      free_events(ctx);
      return hip_fail(ctx, "hipEventCreateWithFlags", e);
    }
  }
  ctx->timing_runs = 0;
  return SV_OK;
}

int spec_verify_set_timing_stride(spec_verify_ctx* ctx, int stride) {
  if (!ctx || stride < 1) return SV_EINVAL;
  ctx->timing_stride = stride;
  ctx->timing_seen = 0;
  return SV_OK;
}

int spec_verify_kernel_times(spec_verify_ctx* ctx, float* ms, const char** names, int cap, int* runs) {
  if (!ctx) return -SV_EINVAL;
  if (runs) *runs = ctx->timing_runs;
  if (ctx->timing_runs == 0) return 0;
  DeviceGuard guard(ctx->device);
  const int R = ctx->timing_runs;
  const PathInfo& path = kPathInfo[ctx->timing_path];
  hipError_t e = hipEventSynchronize(ctx->ev[static_cast<size_t>(R - 1) * kEventsPerRun + 2 * path.nk - 1]);
  if (e != hipSuccess) return -hip_fail(ctx, "hipEventSynchronize", e);
  for (int k = 0; k < path.nk && k < cap; ++k) {
    double sum = 0.0;
    for (int r = 0; r < R; ++r) {
      float t = 0.f;
      hipEvent_t* ev = ctx->ev + static_cast<size_t>(r) * kEventsPerRun;
      e = hipEventElapsedTime(&t, ev[2 * k], ev[2 * k + 1]);
      if (e != hipSuccess) return -hip_fail(ctx, "hipEventElapsedTime", e);
      sum += t;
    }
    if (ms) ms[k] = static_cast<float>(sum / R);
    if (names) names[k] = path.names[k];
  }
  ctx->timing_runs = 0;  // the next runs record afresh
  ctx->timing_seen = 0;
  const int nk = path.nk;
  ctx->timing_path = -1;
  return nk;
}

}  // extern "C"

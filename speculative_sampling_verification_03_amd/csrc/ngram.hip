// Prompt-lookup (n-gram) draft proposer: for every context, find the current suffix
// earlier in the same context and propose the tokens that followed it ("Speculative
// Decoding", atonlee.tistory.com/330, ch.5 prompt lookup; "투기적 디코딩 — 초안 모델을
// 무엇으로 세울 것인가", ailab.paldyn.com, "네 가지 방식" n-gram lookup).
//
// Readings of the rule: suffix lengths n_max .. n_min, the longest that occurs earlier
// wins; "earlier" = the occurrence ends before the last token; of that length the most
// recent occurrence; at most gamma following tokens, fewer where the context ends.
//
// One workgroup per context. Every end position e of a candidate occurrence is judged
// independently: m(e) = the length of the common suffix of c[..e] and c[..L-1], capped at
// n_max; the answer maximises (m(e), e) over m(e) >= n_min. Most positions fail on their
// first token, so the work is one coalesced read of the context. The context is read
// from its end in chunks and the scan stops once a chunk has produced a match of the
// largest possible length: no earlier position can beat it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spec_verify.h"
#include "sv_ngram.h"

namespace {

constexpr int kNgThreads = 256;
constexpr int kNgWaves = kNgThreads / 64;
constexpr int kNgPer = 8;                      // end positions per thread and chunk
constexpr int kNgChunk = kNgThreads * kNgPer;  // positions per chunk
static_assert(SV_NGRAM_MAX_N <= kNgThreads, "the suffix is loaded one token per thread");

__device__ __forceinline__ unsigned long long umax64(unsigned long long x, unsigned long long y) {
  return x > y ? x : y;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = umax64(v, __shfl_xor(v, o));
  return v;
}

__global__ __launch_bounds__(kNgThreads) void k_ngram_propose(NgramArgs a) {
  __shared__ int32_t s_suf[SV_NGRAM_MAX_N];                // s_suf[t] = c[L-1-t]
  __shared__ unsigned long long s_red[2][kNgWaves];         // per-wave maxima, two parities
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t* ids = a.ids + static_cast<size_t>(b) * a.gamma;
  const int c0 = a.cu[b], c1 = a.cu[b + 1];
  if (!(c0 >= 0 && c1 >= c0 && c1 <= a.total)) {  // malformed offsets: no proposal, flagged
    if (tid == 0) {
      atomicOr(a.err, SV_DATA_CONTEXT);
      a.len[b] = 0;
    }
    for (int i = tid; i < a.gamma; i += kNgThreads) ids[i] = -1;
    return;
  }
  const int L = c1 - c0;
  const int32_t* c = a.tok + c0;
  const int nm = min(a.n_max, L - 1);  // longest suffix that can occur earlier
  if (tid < nm) s_suf[tid] = c[L - 1 - tid];
  __syncthreads();

  // key = m << 32 | (e + 1): the maximum is the longest match, then the latest; 0 = none
  unsigned long long best = 0;
  const int e_lo = a.n_min - 1;  // an occurrence of n_min tokens ends at e >= n_min - 1
  if (a.gamma > 0 && nm >= a.n_min) {
    const int32_t last = s_suf[0];
    int par = 0;
    for (int hi = L - 2; hi >= e_lo; hi -= kNgChunk) {  // the same trip count in every thread
      int32_t v[kNgPer];
#pragma unroll
      for (int k = 0; k < kNgPer; ++k) {
        const int e = hi - k * kNgThreads - tid;
        v[k] = e >= e_lo ? c[e] : ~last;
      }
#pragma unroll
      for (int k = 0; k < kNgPer; ++k) {
        if (v[k] != last) continue;  // only positions inside [e_lo, hi] can match
        const int e = hi - k * kNgThreads - tid;
        int m = 1;
        while (m < nm && m <= e && c[e - m] == s_suf[m]) ++m;
        if (m >= a.n_min)
          best = umax64(best, (static_cast<unsigned long long>(m) << 32) | static_cast<unsigned>(e + 1));
      }
      best = wave_max_u64(best);
      if (lane == 0) s_red[par][wave] = best;
      __syncthreads();
#pragma unroll
      for (int w = 0; w < kNgWaves; ++w) best = umax64(best, s_red[par][w]);
      par ^= 1;
      if (static_cast<int>(best >> 32) == nm) break;  // uniform: every thread holds the same best
    }
  }
  const int e = static_cast<int>(best & 0xffffffffu) - 1;
  const int np = best ? min(a.gamma, L - 1 - e) : 0;
  for (int i = tid; i < a.gamma; i += kNgThreads) ids[i] = i < np ? c[e + 1 + i] : -1;
  if (tid == 0) a.len[b] = np;
}

}  // namespace

hipError_t sv_launch_ngram(const NgramArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(k_ngram_propose, dim3(static_cast<unsigned>(a.B)), dim3(kNgThreads), 0, stream, a);
  return hipGetLastError();
}

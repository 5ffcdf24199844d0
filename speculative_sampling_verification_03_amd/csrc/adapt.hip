// Adaptive draft length per sequence ("투기적 디코딩 — 초안 모델을 무엇으로 세울 것인가",
// ailab.paldyn.com, "도입할 때 순서대로 확인할 것": after rejections in a row the draft
// length goes down to 1, while acceptances continue it goes up again; "Speculative
// Decoding", atonlee.tistory.com/330, ch.4: the best length follows the acceptance rate).
//
// Readings of the rule: a round accepts when every draft was accepted and rejects when
// its first draft was rejected; a partly accepted round breaks both runs. up_after
// accepting rounds in a row raise gamma by one (at most gamma_max), down_after rejecting
// rounds in a row cut it to 1; a sequence whose round was not run (accepted count -1)
// keeps its state; a state outside its range is clamped and flagged.
//
// One workgroup updates the whole batch (B <= 65536: a few hundred KB of state) and
// writes the exclusive prefix of the new lengths, the cu_gamma of the next round, so the
// next verification can be enqueued behind it with no host round trip for the layout.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spec_verify.h"
#include "sv_adapt.h"

namespace {

constexpr int kAdThreads = 1024;
constexpr int kAdWaves = kAdThreads / 64;

__device__ __forceinline__ int wave_incl_scan_i(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

__global__ __launch_bounds__(kAdThreads) void k_adapt_gamma(AdaptArgs a) {
  __shared__ int s_w[kAdWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // each thread owns a contiguous run of sequences, so the prefix is one block scan
  const int per = (a.B + kAdThreads - 1) / kAdThreads;
  const int b0 = min(a.B, tid * per), b1 = min(a.B, b0 + per);
  int sum = 0;
  bool bad = false;
  for (int b = b0; b < b1; ++b) {
    int g = a.gamma[b], s = a.streak[b];
    const int n = a.acc[b];
    if (g < 0 || g > a.gmax || s < -a.down || s > a.up) {
      bad = true;
      g = min(max(g, 0), a.gmax);
      s = min(max(s, -a.down), a.up);
    }
    if (n >= 0) {
      if (n >= g) {  // every draft accepted
        s = max(s, 0) + 1;
        if (s >= a.up) {
          g = min(g + 1, a.gmax);
          s = 0;
        }
      } else if (n == 0) {  // the first draft was rejected
        s = min(s, 0) - 1;
        if (-s >= a.down) {
          g = 1;
          s = 0;
        }
      } else {              // some accepted, then a rejection: both runs break
        s = 0;
      }
    }
    a.gamma[b] = g;
    a.streak[b] = s;
    sum += g;
  }
  if (bad) atomicOr(a.err, SV_DATA_STATE);

  const int incl = wave_incl_scan_i(sum, lane);
  if (lane == 63) s_w[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int v = lane < kAdWaves ? s_w[lane] : 0;
    const int vi = wave_incl_scan_i(v, lane);
    if (lane < kAdWaves) s_w[lane] = vi;  // every lane read its entry before this write
  }
  __syncthreads();
  int run = incl - sum + (wave > 0 ? s_w[wave - 1] : 0);
  for (int b = b0; b < b1; ++b) {
    a.cu[b] = run;
    run += a.gamma[b];  // this thread's own store above
  }
  if (tid == kAdThreads - 1) a.cu[a.B] = s_w[kAdWaves - 1];
}

}  // namespace

hipError_t sv_launch_adapt(const AdaptArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(k_adapt_gamma, dim3(1), dim3(kAdThreads), 0, stream, a);
  return hipGetLastError();
}

// Launcher of the prompt-lookup (n-gram) draft proposer, shared between the C ABI in
// spec_verify.hip and the kernel in ngram.hip. Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct NgramArgs {
  const int32_t* tok;  // packed contexts
  const int32_t* cu;   // [B+1] exclusive prefix of the context lengths
  int32_t* ids;        // [B, gamma] proposals, -1 after each one's end
  int32_t* len;        // [B] proposal lengths
  int* err;            // sticky data-error flags
  int B, total, n_min, n_max, gamma;
};

// Enqueues the proposer for a.B > 0 contexts on `stream`; returns the launch status.
__attribute__((visibility("hidden"))) hipError_t sv_launch_ngram(const NgramArgs& a, hipStream_t stream);

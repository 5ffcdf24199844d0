// Launcher of the adaptive draft-length controller, shared between the C ABI in
// spec_verify.hip and the kernel in adapt.hip. Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct AdaptArgs {
  const int32_t* acc;  // [B] accepted counts of the round just verified (-1: not run)
  int32_t* gamma;      // [B] draft lengths, updated in place
  int32_t* streak;     // [B] accepted (> 0) / rejecting (< 0) rounds in a row, in place
  int32_t* cu;         // [B+1] exclusive prefix of the new draft lengths
  int* err;            // sticky data-error flags
  int B, gmax, up, down;
};

constexpr int kAdaptMaxBatch = 65536;

// Enqueues the controller for 0 < a.B <= kAdaptMaxBatch sequences on `stream`.
__attribute__((visibility("hidden"))) hipError_t sv_launch_adapt(const AdaptArgs& a, hipStream_t stream);

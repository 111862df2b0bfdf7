// Internal declarations shared by the host entry points and the kernels'
// launch wrappers.  Not part of the public interface (that is fa_fwd.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Problem description handed from the validated entry point to a launcher.
struct Problem {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N, d;
  float scale;
  int causal;
};

// Each launcher queues its kernel on `stream` and returns the HIP status of
// the launch (hipSuccess or the runtime's error).
hipError_t launch_fwd_f32(const Problem& p, hipStream_t stream);
hipError_t launch_fwd_bf16(const Problem& p, hipStream_t stream);

}  // namespace fa

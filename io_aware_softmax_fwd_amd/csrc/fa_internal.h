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

// Key-split problem: Nq query rows over Nk keys, the keys of every query
// tile cut into `splits` chunks whose partial results go to `workspace`
// (layout in splitkv_layout) before a merge writes o and lse.
struct SplitProblem {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Nq, Nk, d;
  float scale;
  int causal;
  int splits;
  void* workspace;
};

// Workspace layout of the key-split path: partial outputs, fp32
// [splits][B*H*Nq][d], then partial LSEs, fp32 [splits][B*H*Nq], each part
// starting on a 256-byte boundary.
struct SplitLayout {
  int64_t o_bytes, lse_offset, total;
};
inline SplitLayout splitkv_layout(int B, int H, int Nq, int d, int splits) {
  const int64_t rows = (int64_t)B * H * Nq;
  SplitLayout L;
  L.o_bytes = (int64_t)splits * rows * d * 4;
  L.lse_offset = (L.o_bytes + 255) / 256 * 256;
  L.total = L.lse_offset + ((int64_t)splits * rows * 4 + 255) / 256 * 256;
  return L;
}

// Each launcher queues its kernels on `stream` and returns the HIP status of
// the launch (hipSuccess or the runtime's error).
hipError_t launch_fwd_f32(const Problem& p, hipStream_t stream);
hipError_t launch_fwd_bf16(const Problem& p, hipStream_t stream);
hipError_t launch_fwd_bf16_splitkv(const SplitProblem& p, hipStream_t stream);

}  // namespace fa

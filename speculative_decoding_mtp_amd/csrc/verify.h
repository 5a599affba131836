// Host/device interface of the verification kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtp {

constexpr int kTopCap = 2048;   // LDS candidate buffer of the sampling top-k pass
constexpr int kTopSmall = 512;  // second-level candidates ranked by counting
constexpr int kMaxTopK = 128;   // largest top_k on the device path
constexpr int kMaxDraft = 63;   // largest D on the device path

struct VerifyArgs {
  int B, D, V;
  int greedy, q_mode, top_k;
  float temperature, top_p;
  const float* tl;  // target logits [B][D+1][V]
  const float* dl;  // draft logits [B][D][V] (q_mode 1)
  const int32_t* drafts;
  const float *u_accept, *u_sample;
  const int32_t* ctx_len;
  int32_t *n_accept, *out, *crop;
  int nchunk, chunk;
  // greedy scratch
  float* part_v;
  int* part_i;
  // sampling scratch
  float* top_v;  // [rows][top_k]
  int* top_i;
  int* top_n;  // [rows]
};

hipError_t run_verify(const VerifyArgs& a, hipStream_t st);

}  // namespace mtp

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
  int walk;  // greedy: 1 = each workgroup walks its chunk of a sequence's rows in order (early exit)
  // greedy scratch
  float* part_v;
  int* part_i;
  // sampling scratch
  float* top_v;  // [rows][top_k]
  int* top_i;
  int* top_n;  // [rows]
  // few rows: each row in tk_nchunk chunks of tk_chunk items, every chunk's own top-k first
  int tk_nchunk, tk_chunk;
  float* cand_v;  // [rows][tk_nchunk][top_k]
  int* cand_i;
  // the whole vocabulary (top-k off, or larger than the candidate buffer): each row's kept set
  int full;
  struct FullRow* rowinfo;  // [rows]
};

// The kept set of one row under the whole-vocabulary warp: tokens ranked by (logit desc, id asc)
// up to and including the boundary (key, id), where key is the order-preserving bit pattern of
// the logit; weights are exp((l - lmax) / T) in fixed point (2^-40), zk their sum over the set.
struct FullRow {
  float lmax;
  uint32_t key;
  int id;
  int pad;
  unsigned long long zk;
  unsigned long long pad2;
};

// Chunks of the sampling top-k pass: calls with fewer than 128 rows split each row into chunks
// of at least 4096 items (16-byte aligned starts) so that about 512 workgroups stream the logits.
inline void topk_split(int rows, int V, int* nchunk, int* chunk) {
  int n = 1;
  if (rows < 128 && V >= 2 * 4096) {
    n = (512 + rows - 1) / rows;
    if (n > V / 4096) n = V / 4096;
  }
  int c = (V + n - 1) / n;
  c = (c + 3) & ~3;
  *chunk = c;
  *nchunk = (V + c - 1) / c;
}

hipError_t run_verify(const VerifyArgs& a, hipStream_t st);

}  // namespace mtp

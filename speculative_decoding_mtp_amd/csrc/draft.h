// Host/device interface of the draft-head kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mtp.h"

namespace mtp {

constexpr int kLmRows = 16;  // weight rows per lm_head workgroup iteration

constexpr int kMaxSplit = 128;     // attention splits per (sequence, kv head)
constexpr int kMaxGemvGrid = 2048; // workgroups of one GEMV launch (also sizes the lm_head partials)
constexpr int kMaxKSplit = 16;     // K ranges of a split-K MFMA GEMM
constexpr long kPartCols = 98304;  // split-K partial columns per activation row (ksplit x N)
// Calls with more rows per sequence than this (a prefill) count each sequence's valid rows once
// per step into the workspace; shorter ones count them inside every kernel.
constexpr int kInlineRows = 16;

// Positions per attention split for a sequence of T cached positions (a multiple of 64).
__host__ __device__ inline int attn_chunk(int T, int nsplit) {
  int c = (T + nsplit - 1) / nsplit;
  c = (c + 63) & ~63;
  return c < 64 ? 64 : c;
}

struct AttnArgs {
  const float* q;  // [R][nq][hd]
  const void *kc, *vc;
  const int32_t* tok;
  int tok_sb;
  const int32_t* len;
  int B, rps, nq, nkv, max_len, V, nsplit, qstride;
  float* part;       // [B][nkv][nsplit][qstride][hd + 2]
  const int* rows;   // NULL, or the valid rows of sequence b at rows[b]
  float* out;        // set by run_attention: one split of a bf16 cache writes the output rows here
  int shared;        // 1: the rows read a cache they do not append to (keys 0 .. len[b] - 1 only)
  uint16_t *shi, *slo;  // NULL, or where the output rows also go split into bf16 hi + lo, at their
                        // compact row (valid rows of all sequences in order) x nq * hd: the
                        // activations of o_proj on the MFMA path
};

// Arguments of the lm_head finalisation kernel.
struct LmFinal {
  int B;
  const int32_t* tok;
  int tok_sb, rps, V;
  int32_t* len;
  int max_len;
  const float* part_v;  // [B][nparts]
  const int* part_i;
  int nparts;
  const float* x;  // pre-norm residual stream [B * rps][H]
  const void* gain;
  int H;
  float eps;
  float* hout;
  int hout_sb, hout_last;
  int32_t* draft;
  int dr_sb;
  int* status;
  const int* rows;  // NULL, or rows[b] = valid rows, rows[B + b] = the flags that ended them
  int grow;         // 1: len[b] grows by the valid rows (0 for a head reading another model's cache)
};

// Carved out of the caller's workspace.
struct DraftWs {
  int* status;
  int* rows;  // [2B] per-sequence valid rows and flags of many-row calls
  float* x;
  float* q;
  float* attn_part;
  float* attn_out;
  float* act;
  float* lm_part_v;
  int* lm_part_i;
  float* hid_fb;  // [B][D][H] step hiddens when the caller does not want them
  // MFMA path (bf16 heads, 16+ activation rows): compact split-bf16 activations
  uint16_t *xhi, *xlo;  // [R][Kmax]
  int *rowmap, *amap;   // [R]
  int* mcount;
  uint16_t *shi, *slo;  // [R][F] the SwiGLU output split by the gate/up GEMM for down_proj
  float* kpart;    // [kPartCols][R] split-K partial sums
  long kpart_cap;  // floats in kpart
};

struct StepArgs {
  mtp_config cfg;
  const mtp_weights* w;          // the head (target == 0)
  const mtp_target_weights* tw;  // the target (target == 1)
  int target;                    // 1: x = E[tok], logits of every valid row, no draft
  void *kc, *vc;
  int32_t* kv_len;
  int B, max_len, rps, nsplit;
  const int32_t* tok;  // token of (b, i) at tok[b * tok_sb + i]
  int tok_sb;
  const float* hin;  // hidden of (b, i) at hin + (b * hin_sb + i) * H
  int hin_sb;
  float* hout;  // output hidden of (b, i) at hout + (b * hout_sb + (hout_last ? 0 : i)) * H
  int hout_sb, hout_last;
  int32_t* draft;  // draft of b at draft[b * dr_sb]
  int dr_sb;
  float* logits;  // head: NULL or logits of b at logits + b * lg_sb; target: row r at logits + r * V
  long lg_sb;
  DraftWs ws;
  hipStream_t stream;
  hipEvent_t ev_begin, ev_end;  // optional, around the lm_head's main kernel launch
  const char** ev_name;         // set to that kernel's name when the events are recorded
  // A head without a cache of its own: kc/vc/kv_len are the main model's cache, read only; head
  // layer l reads its layer kv_layer[l] (host array); rows sit at kv_len[b] + i + pos_off.
  int shared;
  int pos_off;
  const int32_t* kv_layer;
  int no_head;  // 1: append the rows' K/V and grow len only (no final norm, lm_head or outputs)
};

// Which GEMV layout, variant and grid serve nact activation rows of width K (VE elements per
// 16-byte vector) over N output rows.  kind 0: k_gemv_w with nj = NJ, rw rows per wave; kind 1:
// k_gemv_s with nj = NXM, rw rows per workgroup.  The same plan sizes the lm_head partial buffer
// and launches the kernel.
struct GemvPlan {
  int kind, nj, rb, rw, grid;
};
GemvPlan plan_gemv(int nact, int K, int VE, int N);

int attn_nsplit(int B, int nkv, int max_len, int qrows);
hipError_t run_attention(const AttnArgs& a, int hd, int wdtype, float* out, hipStream_t st);
hipError_t run_step(const StepArgs& s);
hipError_t count_step_rows(const StepArgs& s);  // k_count_rows into s.ws.rows

struct BF16;
struct F32;
template <class W>
hipError_t run_step_t(const StepArgs& s);

}  // namespace mtp

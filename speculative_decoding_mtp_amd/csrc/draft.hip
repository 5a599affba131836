// Host side of the draft step: GEMV layout planning and the weight-type dispatch.
#include "common.h"
#include "draft.h"

namespace mtp {

namespace {
int pow2_at_least(int n) {
  int p = 1;
  while (p < n) p *= 2;
  return p;
}
int pow2_at_most(int n) {
  int p = 1;
  while (p * 2 <= n) p *= 2;
  return p;
}
}  // namespace

// Valid rows of each sequence of a many-row call, counted once per step: the workgroup of sequence b
// scans its tokens together and keeps the first row that ends the prefix (the rule of count_rows),
// writing the count to rows[b] and the flags that ended it to rows[B + b].
// A head reading another model's cache (shared) appends nothing: no capacity limit, but a sequence
// whose cache is empty has no rows.
__global__ __launch_bounds__(kWG) void k_count_rows(const int32_t* tok, int tok_sb, int rps, int V,
                                                    const int32_t* len, int max_len, int B, int shared, int* rows) {
  __shared__ int s_first;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) s_first = rps;
  __syncthreads();
  const int l = len[b];
  const int32_t* t = tok + (long)b * tok_sb;
  for (int i = threadIdx.x; i < rps; i += kWG) {
    const int v = t[i];
    if (v < 0 || v >= V || (shared ? l == 0 : l + i >= max_len)) {  // this thread's first is its least
      atomicMin(&s_first, i);
      break;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int n = s_first;
    int f = 0;
    if (n < rps && t[n] >= 0) f = t[n] >= V ? kFlagToken : (shared ? 0 : kFlagCapacity);
    rows[b] = n;
    rows[B + b] = f;
  }
}

hipError_t count_step_rows(const StepArgs& s) {
  hipLaunchKernelGGL(k_count_rows, dim3(s.B), dim3(kWG), 0, s.stream, s.tok, s.tok_sb, s.rps, s.cfg.vocab, s.kv_len,
                     s.max_len, s.B, s.shared, s.ws.rows);
  return hipGetLastError();
}

GemvPlan plan_gemv(int nact, int K, int VE, int N) {
  const int Kc = K / VE;
  const int nj = (Kc + 63) / 64;
  GemvPlan pl;
  pl.rw = 0;
  // Whole rows per wave while a row is at most 4 loads per lane (K <= 2048 bf16), RW rows per
  // wave and pass with about 8-16 loads in flight.  Wider rows are split over the workgroup: with whole
  // rows, every wave would hold (and normalise) the full activation slice -- 8 loads per lane
  // and row put the wave at one per SIMD, with nothing to overlap its prologue.
  if (nj <= 4) {
    pl.kind = 0;
    pl.nj = pow2_at_least(nj);
    const int rbmax = pl.nj <= 2 ? 4 : 2;
    pl.rb = pow2_at_most(nact < rbmax ? (nact < 1 ? 1 : nact) : rbmax);
    // rows of 4 loads per lane take two rows per wave (8 loads in flight, twice the waves): as
    // fast for the vocabulary-sized lm_head as four, faster for the 2048-column layer matrices
    int rw = pl.nj == 4 ? 2 : 16 / pl.nj;
    // short matrices: fewer rows per wave (down to two) until there are 256+ workgroups
    while (rw > 2 && ((N + rw - 1) / rw + 3) / 4 < 256) rw /= 2;
    pl.rw = rw;
    const int groups = (N + rw - 1) / rw;
    const int wgs = (groups + 3) / 4;
    pl.grid = wgs < kMaxGemvGrid ? wgs : kMaxGemvGrid;
  } else {  // rows split over the workgroup
    pl.kind = 1;
    pl.nj = pow2_at_least((Kc + kWG - 1) / kWG);
    const int rbmax = pl.nj <= 4 ? 4 : 16 / pl.nj;
    pl.rb = pow2_at_most(nact < rbmax ? (nact < 1 ? 1 : nact) : rbmax);
    // rows per workgroup: two for matrices under 4096 rows (1024+ workgroups), else four when
    // eight would leave fewer than 512 workgroups
    pl.rw = (N + 3) / 4 < 1024 ? 2 : ((N + 7) / 8 < 512 ? 4 : 8);
    const int groups = (N + pl.rw - 1) / pl.rw;
    pl.grid = groups < kMaxGemvGrid ? groups : kMaxGemvGrid;
  }
  return pl;
}


hipError_t run_step(const StepArgs& s) {
  return s.cfg.wdtype == MTP_BF16 ? run_step_t<BF16>(s) : run_step_t<F32>(s);
}

}  // namespace mtp

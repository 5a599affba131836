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

GemvPlan plan_gemv(int nact, int K, int VE, int N) {
  const int Kc = K / VE;
  const int nj = (Kc + 63) / 64;
  GemvPlan pl;
  pl.rw = 0;
  if (nj <= 8) {  // whole rows per wave: RW = 16 / NJ rows per pass keep 16 loads in flight
    pl.kind = 0;
    pl.nj = pow2_at_least(nj);
    const int rbmax = pl.nj <= 2 ? 4 : 2;
    pl.rb = pow2_at_most(nact < rbmax ? (nact < 1 ? 1 : nact) : rbmax);
    int rw = 16 / pl.nj;
    // a short matrix with 4 loads per row (fewer than 512 four-wave row groups) takes two rows
    // per wave instead of four
    if (pl.nj == 4 && (N + 4 * rw - 1) / (4 * rw) < 512) rw /= 2;
    pl.rw = rw;
    const int groups = (N + rw - 1) / rw;
    const int wgs = (groups + 3) / 4;
    pl.grid = wgs < kMaxGemvGrid ? wgs : kMaxGemvGrid;
  } else {  // rows split over the workgroup
    pl.kind = 1;
    pl.nj = pow2_at_least((Kc + kWG - 1) / kWG);
    const int rbmax = 16 / pl.nj;
    pl.rb = pow2_at_most(nact < rbmax ? (nact < 1 ? 1 : nact) : rbmax);
    const int groups = (N + 7) / 8;
    pl.grid = groups < kMaxGemvGrid ? groups : kMaxGemvGrid;
  }
  return pl;
}


hipError_t run_step(const StepArgs& s) {
  return s.cfg.wdtype == MTP_BF16 ? run_step_t<BF16>(s) : run_step_t<F32>(s);
}

}  // namespace mtp

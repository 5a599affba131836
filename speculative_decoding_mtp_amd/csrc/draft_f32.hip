// Draft-step kernels for f32 weights (one translation unit per weight type).
#include "draft_impl.h"

namespace mtp {
template hipError_t run_step_t<F32>(const StepArgs& s);
}  // namespace mtp

// Draft-step kernels for bf16 weights (one translation unit per weight type).
#include "draft_impl.h"

namespace mtp {
template hipError_t run_step_t<BF16>(const StepArgs& s);
}  // namespace mtp

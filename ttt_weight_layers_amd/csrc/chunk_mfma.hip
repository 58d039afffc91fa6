// bf16 MFMA chunk kernels (placeholder until the MFMA path lands).
#include "internal.h"

namespace ttt {

bool fast_supported(const Shape&, int) { return false; }

FastPlan fast_plan(const Shape&, int, int) { return FastPlan{}; }

hipError_t launch_fast(const Shape&, const FastPlan&, void*, const FwdArgs&, hipEvent_t, hipEvent_t, int* n) {
    if (n) *n = 0;
    return hipErrorNotSupported;
}

}  // namespace ttt

// Causal prefill over the latent cache on gfx950 (unabsorbed form).  Placeholder until the
// reconstruction GEMM and the causal attention kernel land.
#include "kernels.h"

namespace mla {

bool prefill_supported(const Shape&) { return false; }

PrefillPlan plan_prefill(const Shape&, int, int) { return PrefillPlan{0, 0, 0, 0}; }

hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace mla

// prefill.hip -- causal prefill attention (MFMA path for gfx950).
#include "common.h"
#include "launch.h"

namespace pa {

hipError_t launch_prefill(const PrefillArgs&, Elem, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pa

// Persistent level-ordered decode step (one kernel, device-wide level
// barriers).  Not built yet: the entry points report PWG_ERR_UNSUPPORTED.
#include "pwg_internal.h"

namespace pwg {

size_t step_persistent_workspace(const pwg_step_desc*) { return 0; }

int step_persistent_plan(const pwg_step_desc*, size_t, void*) {
  return fail(PWG_ERR_UNSUPPORTED, "pwg_step_plan: the persistent schedule is not available in this build");
}

int step_persistent_launch(const pwg_step_desc*, size_t, void*) {
  return fail(PWG_ERR_UNSUPPORTED, "pwg_decode_step_weights: the persistent schedule is not available in this build");
}

}  // namespace pwg

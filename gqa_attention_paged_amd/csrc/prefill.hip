// Ragged causal prefill (placeholder until the kernel lands).
#include "dev.hpp"
#include "status.hpp"

using namespace gqap;

extern "C" gqap_status gqap_prefill(const gqap_prefill_plan_t* plan, const void*, const void*, const void*,
                                    const void*, const int32_t*, const uint8_t*, float, void*, float*, void*,
                                    uint64_t, void*) {
  if (!plan || plan->magic != GQAP_PLAN_MAGIC) return fail(GQAP_ERR_INVALID_ARGUMENT, "invalid prefill plan");
  return fail(GQAP_ERR_UNSUPPORTED, "prefill kernel not built");
}

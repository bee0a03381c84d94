// Profilers: interference-free per-op timing (D_best) and pairwise interference (R -> P).
#include "nf_batch.h"
#include "nf_internal.h"

extern "C" nf_status nf_profile_ops(nf_ctx*, const nf_layer_cfg*, const nf_batch_desc*, int32_t, int32_t, int32_t,
                                    const char*) {
  return NF_E_UNSUPPORTED;
}
extern "C" nf_status nf_profile_interference(nf_ctx*, const nf_layer_cfg*, const nf_batch_desc*, int32_t,
                                             const float*, int32_t, const char*) {
  return NF_E_UNSUPPORTED;
}

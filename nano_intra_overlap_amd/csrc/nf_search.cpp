// Two-stage pipeline search.
#include "nf_batch.h"

extern "C" nf_status nf_plan_search(const char*, const char*, const nf_batch_desc*, int32_t, int32_t, char*, size_t) {
  return NF_E_UNSUPPORTED;
}

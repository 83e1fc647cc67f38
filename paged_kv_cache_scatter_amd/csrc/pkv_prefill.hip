// Causal chunked prefill over the paged pool (placeholder until the kernel lands).
#include "pkv_internal.h"

namespace pkv {

bool prefill_supported(int dtype, int head_dim, int rep) {
  (void)dtype;
  (void)head_dim;
  (void)rep;
  return false;
}

pkv_status launch_prefill(const PrefillArgs& a, int dtype, int head_dim, int rep, hipStream_t st) {
  (void)a;
  (void)dtype;
  (void)head_dim;
  (void)rep;
  (void)st;
  set_error("pkv_prefill is not built yet");
  return PKV_ERR_UNSUPPORTED;
}

}  // namespace pkv

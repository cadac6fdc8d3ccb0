#include "decode_latent576.h"

namespace mla {
bool absorb_tuned_applies(const mla_dims&) { return false; }
mla_status launch_absorb_tuned(const mla_dims&, int32_t, const void*, const void*, const int32_t*, const void*,
                               void*, hipStream_t) { return MLA_ERR_UNSUPPORTED; }
bool up_proj_tuned_applies(const mla_dims&) { return false; }
mla_status launch_up_proj_tuned(const mla_dims&, int32_t, const void*, const void*, void*, hipStream_t) {
  return MLA_ERR_UNSUPPORTED;
}
}  // namespace mla

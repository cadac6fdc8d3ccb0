#include "decode_latent576.h"

namespace mla {
bool decode576_supported(const mla_dims&, int32_t) { return false; }
int64_t decode576_default_units(int32_t, int32_t, int cu) { return cu; }
mla_status launch_decode576(const mla_dims&, const DecodePlan&, int32_t, int32_t, const void*, const void*,
                            const int32_t*, int32_t, const int32_t*, void*, void*, float*, hipStream_t) {
  return MLA_ERR_UNSUPPORTED;
}
bool absorb_tuned_applies(const mla_dims&) { return false; }
mla_status launch_absorb_tuned(const mla_dims&, int32_t, const void*, const void*, const int32_t*, const void*,
                               void*, hipStream_t) { return MLA_ERR_UNSUPPORTED; }
bool up_proj_tuned_applies(const mla_dims&) { return false; }
mla_status launch_up_proj_tuned(const mla_dims&, int32_t, const void*, const void*, void*, hipStream_t) {
  return MLA_ERR_UNSUPPORTED;
}
}  // namespace mla

// DeepSeek-V3 shaped bf16 kernels (MFMA).  Placeholder until written.
#include "mla_internal.h"

namespace mla {
bool v3_proj_available() { return false; }

hipError_t launch_absorb_q(const mla_config&, int, const void*, const void*, void*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_out_proj(const mla_config&, int, const void*, const void*, float*, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace mla

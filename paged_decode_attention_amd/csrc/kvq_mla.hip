// kvq_mla.hip -- paged decode over the shared MLA latent slab (gfx950, MFMA).
#include "kvq_internal.h"

namespace kvq {

hipError_t launch_mla_decode(const DecodeArgs&, const DecodePlan&, int, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace kvq

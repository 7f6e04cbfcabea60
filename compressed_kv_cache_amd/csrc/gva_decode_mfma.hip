// Matrix-core decode kernel (bf16 caches).  Placeholder until the kernel
// lands: no shape is routed here yet.
#include "gva_device.h"
#include "gva_internal.h"

namespace gva {

bool mfma_decode_supported(const gva_shape&, bool) { return false; }

DecodePlan plan_mfma_decode(const gva_shape&, int, bool) { return DecodePlan{}; }

hipError_t launch_decode_mfma(const gva_shape&, const DecodePlan&, const DecodeArgs&,
                              hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace gva

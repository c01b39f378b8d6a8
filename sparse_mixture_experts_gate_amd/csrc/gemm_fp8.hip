// FP8 (E4M3) grouped expert GEMMs: placeholder until the MFMA kernel lands.
#include "device_common.h"
#include "internal.h"

namespace dsmoe {

hipError_t launch_ffn_fp8(const FfnArgs&, const GemmTiling&, hipStream_t, hipEvent_t) {
  return hipErrorNotSupported;
}

}  // namespace dsmoe

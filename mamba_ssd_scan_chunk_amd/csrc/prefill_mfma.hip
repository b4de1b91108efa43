// prefill_mfma.hip -- bf16 MFMA prefill (placeholder until the kernels land).
#include "ssd_device.hpp"
#include "ssd_internal.hpp"

namespace ssd {
hipError_t launch_prefill_mfma(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }
}  // namespace ssd

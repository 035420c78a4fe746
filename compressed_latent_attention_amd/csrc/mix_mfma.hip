// placeholder, replaced by the MFMA prefill mix kernel
#include "cca_internal.h"
namespace cca {
bool mix_fwd_mfma_supported(const Dims&) { return false; }
hipError_t launch_mix_fwd_mfma(const MixArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace cca

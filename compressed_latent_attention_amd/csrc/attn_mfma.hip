// placeholder, replaced by the MFMA flash-attention kernel
#include "cca_internal.h"
namespace cca {
bool attn_fwd_mfma_supported(const Dims&) { return false; }
hipError_t launch_attn_fwd_mfma(const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace cca

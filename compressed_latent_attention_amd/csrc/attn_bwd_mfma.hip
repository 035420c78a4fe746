// placeholder, replaced by the MFMA attention backward kernels
#include "cca_internal.h"
namespace cca {
bool attn_bwd_mfma_supported(const Dims&) { return false; }
hipError_t launch_attn_bwd_mfma(const AttnBwdArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace cca

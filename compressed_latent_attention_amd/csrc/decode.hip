// placeholder decode attention: routes to the generic kernel
#include "cca_internal.h"
namespace cca {
int decode_nsplit(const Dims&, int) { return 1; }
size_t decode_part_floats(const Dims&, int) { return 0; }
hipError_t launch_attn_decode(const AttnArgs& a, hipStream_t s) { return launch_attn_fwd(a, s); }
}  // namespace cca

// Backward kernels of the GDN chunked prefill (gfx950).
#include "gdn_common.hpp"
#include "gdn_internal.h"

namespace gdn {

hipError_t launch_bwd(const BwdArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace gdn

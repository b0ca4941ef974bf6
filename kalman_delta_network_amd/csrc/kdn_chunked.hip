// kdn_chunked.hip -- chunkwise WY/UT forward on gfx950 matrix cores.
#include "kdn_internal.h"

namespace kdn {

bool chunked_supports(const FwdArgs&) { return false; }

hipError_t launch_chunked(const FwdArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace kdn

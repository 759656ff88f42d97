// Forward-kernel instantiations for bf16 io.
#include "ssd_fwd_launch.h"

namespace ssd {
bool fwd_dispatch_bf16(SSD_FWD_PARAMS) { return fwd_dispatch<bf16>(SSD_FWD_ARGS); }
}  // namespace ssd

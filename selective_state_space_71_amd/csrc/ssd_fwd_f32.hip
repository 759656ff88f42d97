// Forward-kernel instantiations for fp32 io.
#include "ssd_fwd_launch.h"

namespace ssd {
bool fwd_dispatch_f32(SSD_FWD_PARAMS) { return fwd_dispatch<float>(SSD_FWD_ARGS); }
}  // namespace ssd

// Forward-kernel instantiations for fp32 io.
#include "ssd_fwd_launch.h"

namespace ssd {
bool fwd_dispatch_f32(int p, int n, int q, const FwdParams &prm, unsigned grid, hipStream_t st,
                      bool launch, hipError_t *err) {
    return fwd_dispatch<float>(p, n, q, prm, grid, st, launch, err);
}
}  // namespace ssd

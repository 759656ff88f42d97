// Forward-kernel instantiations for bf16 io.
#include "ssd_fwd_launch.h"

namespace ssd {
bool fwd_dispatch_bf16(int p, int n, int q, const FwdParams &prm, unsigned grid, hipStream_t st,
                       bool launch, hipError_t *err) {
    return fwd_dispatch<bf16>(p, n, q, prm, grid, st, launch, err);
}
}  // namespace ssd

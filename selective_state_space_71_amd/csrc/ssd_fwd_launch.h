// ssd_fwd_launch.h -- instantiation and dispatch of the forward kernel over
// the supported (headdim, dstate, chunk_len) shapes of one io dtype.
#pragma once

#include "ssd_fwd_kernel.h"

namespace ssd {

// Launches one workgroup per possible work item (chunk entry, group, head
// slice), rounded up to a multiple of the XCD count; workgroups loop over
// their XCD's item list.  Returns true when the shape is built; launches only
// if `launch`.
template <typename IO, int P, int N, int Q>
static bool fwd_try(int p, int n, int qq, const FwdParams &prm, long long max_entries, hipStream_t st,
                    bool launch, hipError_t *err) {
    if (p != P || n != N || qq != Q) return false;
    if constexpr (FwdShape<IO, P, N, Q>::kFits) {
        if (launch) {
            long long blocks = max_entries * prm.G * prm.slices;
            blocks = (blocks + prm.n_xcd - 1) / prm.n_xcd * prm.n_xcd;
            hipLaunchKernelGGL((ssd_fwd_kernel<IO, P, N, Q>), dim3((unsigned)blocks),
                               dim3(FwdShape<IO, P, N, Q>::kThreads), 0, st, prm);
            *err = hipGetLastError();
        }
        return true;
    } else {
        return false;
    }
}

#define SSD_FWD_ARGS p, n, q, prm, max_entries, st, launch, err
#define SSD_FWD_PARAMS int p, int n, int q, const FwdParams &prm, long long max_entries, hipStream_t st, \
                       bool launch, hipError_t *err

template <typename IO, int P, int N>
static bool fwd_try_q(SSD_FWD_PARAMS) {
    return fwd_try<IO, P, N, 64>(SSD_FWD_ARGS) || fwd_try<IO, P, N, 128>(SSD_FWD_ARGS) ||
           fwd_try<IO, P, N, 256>(SSD_FWD_ARGS);
}

template <typename IO, int P>
static bool fwd_try_n(SSD_FWD_PARAMS) {
    return fwd_try_q<IO, P, 16>(SSD_FWD_ARGS) || fwd_try_q<IO, P, 32>(SSD_FWD_ARGS) ||
           fwd_try_q<IO, P, 64>(SSD_FWD_ARGS) || fwd_try_q<IO, P, 128>(SSD_FWD_ARGS) ||
           fwd_try_q<IO, P, 256>(SSD_FWD_ARGS);
}

// Kernel head dims 16, 32 and 64 (head dim 128 runs as two kernel heads of 64).
template <typename IO>
static bool fwd_dispatch(SSD_FWD_PARAMS) {
    return fwd_try_n<IO, 16>(SSD_FWD_ARGS) || fwd_try_n<IO, 32>(SSD_FWD_ARGS) || fwd_try_n<IO, 64>(SSD_FWD_ARGS);
}

}  // namespace ssd

// ssd_fwd_launch.h -- instantiation and dispatch of the forward kernel over
// the supported (headdim, dstate, chunk_len) shapes of one io dtype.
#pragma once

#include "ssd_fwd_kernel.h"

namespace ssd {

template <typename IO, int P, int N, int Q>
static bool fwd_try(int p, int n, int qq, const FwdParams &prm, unsigned grid, hipStream_t st,
                    bool launch, hipError_t *err) {
    if (p != P || n != N || qq != Q) return false;
    if constexpr (FwdShape<IO, P, N, Q>::kFits) {
        if (launch) {
            hipLaunchKernelGGL((ssd_fwd_kernel<IO, P, N, Q>), dim3(grid), dim3(FwdShape<IO, P, N, Q>::kThreads), 0, st, prm);
            *err = hipGetLastError();
        }
        return true;
    } else {
        return false;
    }
}

template <typename IO, int P, int N>
static bool fwd_try_q(int p, int n, int q, const FwdParams &prm, unsigned grid, hipStream_t st,
                      bool launch, hipError_t *err) {
    return fwd_try<IO, P, N, 64>(p, n, q, prm, grid, st, launch, err) ||
           fwd_try<IO, P, N, 128>(p, n, q, prm, grid, st, launch, err) ||
           fwd_try<IO, P, N, 256>(p, n, q, prm, grid, st, launch, err);
}

template <typename IO, int P>
static bool fwd_try_n(int p, int n, int q, const FwdParams &prm, unsigned grid, hipStream_t st,
                      bool launch, hipError_t *err) {
    return fwd_try_q<IO, P, 16>(p, n, q, prm, grid, st, launch, err) ||
           fwd_try_q<IO, P, 32>(p, n, q, prm, grid, st, launch, err) ||
           fwd_try_q<IO, P, 64>(p, n, q, prm, grid, st, launch, err) ||
           fwd_try_q<IO, P, 128>(p, n, q, prm, grid, st, launch, err);
}

// Returns true when the shape is built; launches when `launch` is set.
template <typename IO>
static bool fwd_dispatch(int p, int n, int q, const FwdParams &prm, unsigned grid, hipStream_t st,
                         bool launch, hipError_t *err) {
    return fwd_try_n<IO, 16>(p, n, q, prm, grid, st, launch, err) ||
           fwd_try_n<IO, 32>(p, n, q, prm, grid, st, launch, err) ||
           fwd_try_n<IO, 64>(p, n, q, prm, grid, st, launch, err);
}

}  // namespace ssd

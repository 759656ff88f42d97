// ssd_fwd_kernel.h -- fused chunked SSD forward kernel for gfx950.
//
// Algorithm ("Transformers are SSMs Review", section 3-2(4): split the
// sequence into chunks, evaluate the diagonal blocks in the quadratic masked
// form, carry chunk-boundary states between chunks, fold them back into the
// outputs).  Per (sequence, head h, chunk c) with in-chunk index i in [0, q),
// a_t = dt_t A_h and s_i the inclusive in-chunk cumulative sum of a:
//   Y_diag = (C B^T o Lambda) diag(dt) X,   Lambda_ij = exp(s_i - s_j), j <= i
//   S_c    = X^T diag(exp(s_{q-1} - s_j) dt_j) B         (chunk state from 0)
//   H_{c+1} = exp(s_{q-1}) H_c + S_c                     (inter-chunk recurrence)
//   Y_off  = diag(exp(s_i)) C H_c^T
//   y      = Y_diag + Y_off + D_h x
//
// One workgroup (4 waves) owns one (chunk, head).  Workgroups take a ticket
// from a global counter; tickets are ordered chunk-index-major, so the
// workgroup holding chunk c-1 of the same (sequence, head) always started
// earlier.  Each workgroup computes S_c first, then waits for its
// predecessor's boundary state (a progress flag per (sequence, head)),
// publishes H_{c+1} and only then computes the outputs, so the serial chain
// carries just a P x N fp32 state per link.  The state buffer is the caller's
// final_state (or workspace): after the last chunk it holds the final state.
//
// LDS (per workgroup): B chunk [Q][N] (row layout), x^T scaled by dt and by
// the chunk-end decay (two [P][Q] copies; the second is reused for the
// incoming state as io), and per-token s, dt, exp(s).
#pragma once

#include "ssd_device.h"

namespace ssd {

struct FwdParams {
    const void *x;
    const float *dt;
    const float *A;
    const void *B;
    const void *C;
    const float *D;           // may be null
    const float *init_state;  // may be null
    void *y;
    float *state;             // boundary-state buffer; holds the final state at the end
    const int4 *chunks;       // {seq, chunk index in seq, first token, length}
    const int *n_chunks;      // number of valid chunk entries
    int *ticket;
    int *flags;               // per (sequence, head): chunks whose state is published
    int *error;
    int H, G;
    long long grid;           // workgroups launched
};

template <int v> struct IntC { static constexpr int value = v; };
constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <typename IO, int P, int N, int Q>
struct FwdShape {
    static constexpr int kThreads = 256;
    static constexpr int kWaves = 4;
    static constexpr int PT = P / 16;            // 16-wide tiles over the head dim
    static constexpr int NT = N / 16;            // 16-wide tiles over the state dim
    static constexpr int NK = (N + 31) / 32;     // K steps over the state dim
    static constexpr int NP = NK * 32;           // state dim padded to a K step
    static constexpr int QT = Q / 16;            // 16-row tiles of a chunk
    static constexpr int QK = Q / 32;            // K steps over a chunk
    static constexpr int NTW = (NT + kWaves - 1) / kWaves;  // state tiles per wave
    static constexpr int E = (int)sizeof(IO);
    static constexpr int PAD = 16 / E;           // 16 bytes of padding per LDS row
    static constexpr int SB = NP + PAD;          // row stride of the B tile
    static constexpr int SX = Q + PAD;           // row stride of the x^T tiles
    static constexpr int SH = NP + PAD;          // row stride of the incoming state
    static constexpr int kLdsB = Q * SB * E;
    static constexpr int kLdsXd = P * SX * E;
    static constexpr int kLdsXw = cmax(P * SX, P * SH) * E;
    static constexpr int kLdsScal = 3 * Q * 4;
    static constexpr int kLds = kLdsB + kLdsXd + kLdsXw + kLdsScal + 16;
    static constexpr bool kFits = kLds <= 160 * 1024;
};

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Row tile handled by `wave` in its round `k`: a snake order over the waves,
// so that every wave gets a similar share of the causal (triangular) work.
__device__ __forceinline__ int snake_tile(int wave, int k, int nwaves) {
    const int blk = k;
    return blk * nwaves + ((blk & 1) ? (nwaves - 1 - wave) : wave);
}

template <typename IO, int P, int N, int Q>
__global__ __launch_bounds__(256) void ssd_fwd_kernel(FwdParams prm) {
    typedef FwdShape<IO, P, N, Q> S;
    typedef typename Io<IO>::Frag Frag;
    static_assert(S::kFits, "chunk tiles do not fit in LDS");

    __shared__ __attribute__((aligned(16))) char smem[S::kLds];
    IO *sB = reinterpret_cast<IO *>(smem);
    IO *sXd = reinterpret_cast<IO *>(smem + S::kLdsB);
    IO *sXw = reinterpret_cast<IO *>(smem + S::kLdsB + S::kLdsXd);
    IO *sH = sXw;  // reused once the chunk state is formed
    float *sS = reinterpret_cast<float *>(smem + S::kLdsB + S::kLdsXd + S::kLdsXw);
    float *sDt = sS + Q;
    float *sE = sDt + Q;
    int *sTicket = reinterpret_cast<int *>(sE + Q);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int li = lane & 15;
    const int lg = lane >> 4;

    if (tid == 0) sTicket[0] = atomicAdd(prm.ticket, 1);
    __syncthreads();
    const int ticket = sTicket[0];
    const int H = prm.H;
    const int entry = ticket / H;
    const int h = ticket - entry * H;
    if (entry >= *prm.n_chunks) return;
    const int4 ce = prm.chunks[entry];
    const int seq = ce.x;
    const int cloc = ce.y;
    const long long tok0 = ce.z;
    const int q = ce.w;
    const int G = prm.G;
    const int g = h / (H / G);
    const float Ah = prm.A[h];
    const float Dh = prm.D ? prm.D[h] : 0.f;
    const long long xs = (long long)H * P;   // token stride of x and y
    const long long bs = (long long)G * N;   // token stride of B and C
    const IO *xg = reinterpret_cast<const IO *>(prm.x) + tok0 * xs + (long long)h * P;
    const IO *Bg = reinterpret_cast<const IO *>(prm.B) + tok0 * bs + (long long)g * N;
    const IO *Cg = reinterpret_cast<const IO *>(prm.C) + tok0 * bs + (long long)g * N;
    IO *yg = reinterpret_cast<IO *>(prm.y) + tok0 * xs + (long long)h * P;
    const float *dtg = prm.dt + tok0 * H + h;

    // ---- in-chunk cumulative sum of dt*A (wave 0, one wave-wide scan) ----
    if (wave == 0) {
        constexpr int R = Q / 64;
        float a[R];
        float run = 0.f;
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int i = lane * R + k;
            const float d = (i < q) ? dtg[(long long)i * H] : 0.f;
            sDt[i] = d;
            run += d * Ah;
            a[k] = run;
        }
        float incl = run;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float v = __shfl_up(incl, off, 64);
            if (lane >= off) incl += v;
        }
        const float excl = incl - run;
#pragma unroll
        for (int k = 0; k < R; ++k) sS[lane * R + k] = excl + a[k];
    }
    __syncthreads();
    const float s_last = sS[Q - 1];
    for (int i = tid; i < Q; i += S::kThreads) sE[i] = __expf(sS[i]);

    // ---- stage the B chunk, row layout [j][n], zero outside the chunk ----
    {
        constexpr int VPR = S::NP * S::E / 16;  // 16-byte vectors per LDS row
        constexpr int VN = N * S::E / 16;       // vectors that hold data
        for (int v = tid; v < Q * VPR; v += S::kThreads) {
            const int j = v / VPR;
            const int c = v - j * VPR;
            i32x4 val = {0, 0, 0, 0};
            if (j < q && c < VN)
                val = *reinterpret_cast<const i32x4 *>(Bg + (long long)j * bs + c * (16 / S::E));
            *reinterpret_cast<i32x4 *>(sB + j * S::SB + c * (16 / S::E)) = val;
        }
    }
    // ---- stage x^T scaled by dt (sXd) and by the chunk-end decay (sXw) ----
    {
        constexpr int PB = P / 8;
        for (int u = tid; u < (Q / 2) * PB; u += S::kThreads) {
            const int ip = u / PB;
            const int p0 = (u - ip * PB) * 8;
            const int i0 = 2 * ip;
            float v0[8], v1[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) { v0[e] = 0.f; v1[e] = 0.f; }
            if (i0 < q) {
#pragma unroll
                for (int e = 0; e < 8; ++e) v0[e] = to_f32(xg[(long long)i0 * xs + p0 + e]);
            }
            if (i0 + 1 < q) {
#pragma unroll
                for (int e = 0; e < 8; ++e) v1[e] = to_f32(xg[(long long)(i0 + 1) * xs + p0 + e]);
            }
            const float d0 = sDt[i0], d1 = sDt[i0 + 1];
            const float w0 = __expf(s_last - sS[i0]) * d0;
            const float w1 = __expf(s_last - sS[i0 + 1]) * d1;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                IO *pd = sXd + (p0 + e) * S::SX + i0;
                IO *pw = sXw + (p0 + e) * S::SX + i0;
                pd[0] = from_f32<IO>(v0[e] * d0);
                pd[1] = from_f32<IO>(v1[e] * d1);
                pw[0] = from_f32<IO>(v0[e] * w0);
                pw[1] = from_f32<IO>(v1[e] * w1);
            }
        }
    }
    __syncthreads();

    // ---- chunk state S_c = (x w)^T B : P x N, K = chunk tokens ----
    f32x4 accS[S::NTW][S::PT];
#pragma unroll
    for (int a = 0; a < S::NTW; ++a)
#pragma unroll
        for (int b = 0; b < S::PT; ++b) accS[a][b] = zero4();
#pragma unroll 1
    for (int ks = 0; ks < S::QK; ++ks) {
        Frag af[S::PT];
#pragma unroll
        for (int pt = 0; pt < S::PT; ++pt)
            af[pt] = *reinterpret_cast<const Frag *>(sXw + (pt * 16 + li) * S::SX + ks * 32 + 8 * lg);
#pragma unroll
        for (int a = 0; a < S::NTW; ++a) {
            const int nt = wave + a * S::kWaves;
            if (nt < S::NT) {
                Frag bfr;
                if constexpr (sizeof(IO) == 2) {
                    const int row = ks * 32 + 8 * lg + (li >> 2);
                    const int col = nt * 16 + 4 * (li & 3);
                    const bf16x4 lo = lds_read_tr16(reinterpret_cast<const bf16 *>(sB + row * S::SB + col));
                    const bf16x4 hi = lds_read_tr16(reinterpret_cast<const bf16 *>(sB + (row + 4) * S::SB + col));
                    bfr = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) bfr[e] = sB[(ks * 32 + 8 * lg + e) * S::SB + nt * 16 + li];
                }
#pragma unroll
                for (int pt = 0; pt < S::PT; ++pt) accS[a][pt] = Io<IO>::mfma(accS[a][pt], af[pt], bfr);
            }
        }
    }
    __syncthreads();  // sXw is about to be overwritten with the incoming state

    // ---- wait for the incoming boundary state, publish the outgoing one ----
    const int unit = seq * H + h;
    if (cloc > 0) {
        if (tid == 0) {
            int it = 0;
            while (__hip_atomic_load(prm.flags + unit, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < cloc) {
                __builtin_amdgcn_s_sleep(2);
                if (++it > (1 << 22)) {
                    atomicOr(prm.error, 1);
                    break;
                }
            }
        }
        __syncthreads();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    const float *hin = (cloc == 0) ? (prm.init_state ? prm.init_state + (long long)unit * P * N : nullptr)
                                   : prm.state + (long long)unit * P * N;
    float *hout = prm.state + (long long)unit * P * N;
    const float alpha = __expf(s_last);
    if constexpr (S::NP != N) {
        for (int v = tid; v < P * (S::NP - N); v += S::kThreads) {
            const int p = v / (S::NP - N);
            sH[p * S::SH + N + (v - p * (S::NP - N))] = from_f32<IO>(0.f);
        }
    }
#pragma unroll
    for (int a = 0; a < S::NTW; ++a) {
        const int nt = wave + a * S::kWaves;
        if (nt < S::NT) {
#pragma unroll
            for (int pt = 0; pt < S::PT; ++pt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int p = pt * 16 + 4 * lg + r;
                    const int n = nt * 16 + li;
                    const float hv = hin ? hin[p * N + n] : 0.f;
                    hout[p * N + n] = alpha * hv + accS[a][pt][r];
                    sH[p * S::SH + n] = from_f32<IO>(hv);
                }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (tid == 0)
        __hip_atomic_store(prm.flags + unit, cloc + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);

    // ---- outputs, one 16-row tile at a time ----
#pragma unroll 1
    for (int k = 0;; ++k) {
        const int I = snake_tile(wave, k, S::kWaves);
        if (I >= S::QT) break;
        const int i0 = I * 16;
        if (i0 >= q) continue;
        // C rows as fragments (B operand of C B^T, A operand of C H^T)
        Frag cf[S::NK];
        {
            const int i = i0 + li;
#pragma unroll
            for (int ks = 0; ks < S::NK; ++ks) {
                const int n0 = ks * 32 + 8 * lg;
                if (i < q && n0 < N)
                    cf[ks] = *reinterpret_cast<const Frag *>(Cg + (long long)i * bs + n0);
                else
                    cf[ks] = zero_frag<Frag>();
            }
        }
        f32x4 accO[S::PT], accY[S::PT];
#pragma unroll
        for (int pt = 0; pt < S::PT; ++pt) { accO[pt] = zero4(); accY[pt] = zero4(); }
        // state read-out: C H^T
#pragma unroll
        for (int ks = 0; ks < S::NK; ++ks)
#pragma unroll
            for (int pt = 0; pt < S::PT; ++pt) {
                const Frag hf = *reinterpret_cast<const Frag *>(sH + (pt * 16 + li) * S::SH + ks * 32 + 8 * lg);
                accO[pt] = Io<IO>::mfma(accO[pt], cf[ks], hf);
            }
        // diagonal block: (C B^T o Lambda) (dt x)
        const float s_i = sS[i0 + li];
        const int i_row = i0 + li;
#pragma unroll 1
        for (int kj = 0; kj <= I / 2; ++kj) {
            f32x4 gt[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int jt = 2 * kj + half;
                gt[half] = zero4();
                if (jt <= I) {
#pragma unroll
                    for (int ks = 0; ks < S::NK; ++ks) {
                        const Frag bfr = *reinterpret_cast<const Frag *>(sB + (jt * 16 + li) * S::SB + ks * 32 + 8 * lg);
                        gt[half] = Io<IO>::mfma(gt[half], bfr, cf[ks]);
                    }
                }
            }
            Frag m;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int half = e >> 2;
                const int j = 32 * kj + 16 * half + 4 * lg + (e & 3);
                const float v = (j <= i_row) ? gt[half][e & 3] * __expf(s_i - sS[j]) : 0.f;
                m[e] = from_f32<IO>(v);
            }
#pragma unroll
            for (int pt = 0; pt < S::PT; ++pt) {
                const IO *xr = sXd + (pt * 16 + li) * S::SX + 32 * kj + 4 * lg;
                typedef typename Io<IO>::Half Half;
                const Half lo = *reinterpret_cast<const Half *>(xr);
                const Half hi = *reinterpret_cast<const Half *>(xr + 16);
                const Frag xf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                accY[pt] = Io<IO>::mfma(accY[pt], m, xf);
            }
        }
        // y = Y_diag + exp(s_i) Y_off + D x
#pragma unroll
        for (int pt = 0; pt < S::PT; ++pt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = i0 + 4 * lg + r;
                if (i < q) {
                    const int p = pt * 16 + li;
                    const float xv = to_f32(xg[(long long)i * xs + p]);
                    const float yv = accY[pt][r] + sE[i] * accO[pt][r] + Dh * xv;
                    yg[(long long)i * xs + p] = from_f32<IO>(yv);
                }
            }
    }
}

}  // namespace ssd

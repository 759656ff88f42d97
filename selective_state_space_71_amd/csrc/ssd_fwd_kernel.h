// ssd_fwd_kernel.h -- fused chunked SSD forward kernel for gfx950.
//
// Algorithm ("Transformers are SSMs Review", section 3-2(4): split the
// sequence into chunks, evaluate the diagonal blocks in the quadratic masked
// form, carry chunk-boundary states between chunks, fold them back into the
// outputs).  Per (sequence, head h, chunk c) with in-chunk index i in [0, q),
// a_t = dt_t A_h and s_i the inclusive in-chunk cumulative sum of a:
//   Y_diag  = (C B^T o Lambda) diag(dt) X,   Lambda_ij = exp(s_i - s_j), j <= i
//   S_c     = X^T diag(exp(s_{q-1} - s_j) dt_j) B        (chunk state from 0)
//   H_{c+1} = exp(s_{q-1}) H_c + S_c                     (inter-chunk recurrence)
//   Y_off   = diag(exp(s_i)) C H_c^T
//   y       = Y_diag + Y_off + D_h x
//
// Scheduling.  One workgroup (8 waves) owns one (chunk, head).  Workgroups
// take a ticket from a global counter; tickets are ordered chunk-index-major,
// so the workgroup holding chunk c-1 of the same (sequence, head) always
// started earlier and the chain cannot deadlock.  Each workgroup forms S_c
// first, then waits for its predecessor's boundary state (a progress flag per
// (sequence, head)), publishes H_{c+1}, and only then computes the outputs:
// the serial chain carries one P x N fp32 state per link.  The state buffer is
// the caller's final_state (or workspace) and ends up holding the final state.
//
// Numerics.  All decays are products of factors <= 1 (A <= 0, dt >= 0):
// for a 16 x 16 tile (I, J) below the diagonal,
//   exp(s_i - s_j) = exp(s_i - s_r) * exp(s_r - s_j),  r = last token of tile J,
// so only the diagonal tiles need a per-element exponential; the chunk-state
// weights exp(s_{q-1} - s_j) and the read-out weights exp(s_i) are per-token
// vectors.  Exponentials are evaluated as exp2 of log2(e)-scaled sums.
//
// LDS: the B chunk [Q][N] (row layout; transposed fragments come from the
// gfx950 transposing LDS read), the raw x chunk transposed [P][Q], the
// incoming state as io [P][N], and per-token vectors.
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
};

constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int cmin(int a, int b) { return a < b ? a : b; }

template <typename IO, int P, int N, int Q>
struct FwdShape {
    static constexpr int kWaves = 8;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int PT = P / 16;            // 16-wide tiles over the head dim
    static constexpr int NT = N / 16;            // 16-wide tiles over the state dim
    static constexpr int NK = (N + 31) / 32;     // K steps over the state dim
    static constexpr int NP = NK * 32;           // state dim padded to a K step
    static constexpr int QT = Q / 16;            // 16-row tiles of a chunk
    static constexpr int QK = Q / 32;            // K steps over a chunk
    // chunk-state work split: WN waves along the state dim, WP along the head dim
    static constexpr int WN = cmin(NT, kWaves);
    static constexpr int WP = kWaves / WN;
    static constexpr int NTW = (NT + WN - 1) / WN;   // state tiles per wave
    static constexpr int PTW = (PT + WP - 1) / WP;   // head-dim tiles per wave
    static constexpr int E = (int)sizeof(IO);
    static constexpr int PAD = 16 / E;           // 16 bytes of padding per LDS row
    static constexpr int SB = NP + PAD;          // row stride of the B tile
    static constexpr int SX = Q + PAD;           // row stride of the x^T tile
    static constexpr int SH = NP + PAD;          // row stride of the incoming state
    static constexpr int kLdsB = Q * SB * E;
    static constexpr int kLdsX = P * SX * E;
    static constexpr int kLdsH = P * SH * E;
    static constexpr int kNVec = 6;              // per-token float vectors
    static constexpr int kLdsVec = kNVec * Q * 4;
    static constexpr int kLds = kLdsB + kLdsX + kLdsH + kLdsVec + 16;
    static constexpr bool kFits = kLds <= 160 * 1024;
};

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2f_fast(float v) { return __builtin_amdgcn_exp2f(v); }

// Row tile handled by `wave` in its round `k`: a snake order over the waves,
// so that every wave gets a similar share of the causal (triangular) work.
__device__ __forceinline__ int snake_tile(int wave, int k, int nwaves) {
    return k * nwaves + ((k & 1) ? (nwaves - 1 - wave) : wave);
}

// Unscaled B^T fragment: lane holds B[k0 + 8*lg + e][n0 + li], e = 0..7.
template <typename IO, int SB>
__device__ __forceinline__ typename Io<IO>::Frag load_bt_frag(const IO *sB, int k0, int n0, int li, int lg) {
    typename Io<IO>::Frag f;
    if constexpr (sizeof(IO) == 2) {
        const int row = k0 + 8 * lg + (li >> 2);
        const int col = n0 + 4 * (li & 3);
        const bf16x4 lo = lds_read_tr16(reinterpret_cast<const bf16 *>(sB + row * SB + col));
        const bf16x4 hi = lds_read_tr16(reinterpret_cast<const bf16 *>(sB + (row + 4) * SB + col));
        f = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = sB[(k0 + 8 * lg + e) * SB + n0 + li];
    }
    return f;
}

// Slot-wise scaling of a fragment: slot e by lo[e] (e < 4) or hi[e - 4].
template <typename IO>
__device__ __forceinline__ typename Io<IO>::Frag scale_frag(typename Io<IO>::Frag f, f32x4 lo, f32x4 hi) {
    typename Io<IO>::Frag o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        o[e] = from_f32<IO>(to_f32(f[e]) * lo[e]);
        o[e + 4] = from_f32<IO>(to_f32(f[e + 4]) * hi[e]);
    }
    return o;
}

template <typename IO, int P, int N, int Q>
__global__ __launch_bounds__(512) void ssd_fwd_kernel(FwdParams prm) {
    typedef FwdShape<IO, P, N, Q> S;
    typedef typename Io<IO>::Frag Frag;
    typedef typename Io<IO>::Half Half;
    static_assert(S::kFits, "chunk tiles do not fit in LDS");

    __shared__ __attribute__((aligned(16))) char smem[S::kLds];
    IO *sB = reinterpret_cast<IO *>(smem);
    IO *sX = reinterpret_cast<IO *>(smem + S::kLdsB);
    IO *sH = reinterpret_cast<IO *>(smem + S::kLdsB + S::kLdsX);
    float *vS2 = reinterpret_cast<float *>(smem + S::kLdsB + S::kLdsX + S::kLdsH);  // s * log2(e)
    float *vDt = vS2 + Q;     // dt_j
    float *vCol = vDt + Q;    // exp(s_r - s_j) dt_j, r = last token of j's 16-tile
    float *vW = vCol + Q;     // exp(s_last - s_j) dt_j
    float *vEo = vW + Q;      // exp(s_i)
    float *vRef = vEo + Q;    // s2 of the last token of each 16-tile (QT used)
    int *sTicket = reinterpret_cast<int *>(vRef + Q);

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
    const int xs = H * P;    // token stride of x and y (elements)
    const int bs = G * N;    // token stride of B and C
    const IO *xg = reinterpret_cast<const IO *>(prm.x) + tok0 * xs + h * P;
    const IO *Bg = reinterpret_cast<const IO *>(prm.B) + tok0 * bs + g * N;
    const IO *Cg = reinterpret_cast<const IO *>(prm.C) + tok0 * bs + g * N;
    IO *yg = reinterpret_cast<IO *>(prm.y) + tok0 * xs + h * P;
    const float *dtg = prm.dt + tok0 * H + h;

    // ---- issue the global loads of the B and x chunks early ----
    constexpr int VPR = S::NP * S::E / 16;          // 16-byte vectors per B row in LDS
    constexpr int VN = N * S::E / 16;               // vectors that hold data
    constexpr int NVB = (Q * VPR + S::kThreads - 1) / S::kThreads;
    i32x4 bval[NVB];
#pragma unroll
    for (int k = 0; k < NVB; ++k) {
        const int v = tid + k * S::kThreads;
        const int j = v / VPR;
        const int c = v - j * VPR;
        bval[k] = i32x4{0, 0, 0, 0};
        if (v < Q * VPR && j < q && c < VN)
            bval[k] = *reinterpret_cast<const i32x4 *>(Bg + j * bs + c * (16 / S::E));
    }
    // x: a unit is 4 consecutive tokens x 8 channels
    constexpr int PB = P / 8;
    constexpr int NUNIT = (Q / 4) * PB;
    constexpr int NU = (NUNIT + S::kThreads - 1) / S::kThreads;
    Frag xr[NU][4];
#pragma unroll
    for (int k = 0; k < NU; ++k) {
        const int u = tid + k * S::kThreads;
        const int it = u / PB;
        const int p0 = (u - it * PB) * 8;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int i = 4 * it + t;
            xr[k][t] = zero_frag<Frag>();
            if (u < NUNIT && i < q) xr[k][t] = *reinterpret_cast<const Frag *>(xg + i * xs + p0);
        }
    }

    // ---- in-chunk cumulative sum of dt*A (wave 0) and per-token vectors ----
    if (wave == 0) {
        constexpr int R = Q / 64;
        float a[R];
        float run = 0.f;
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int i = lane * R + k;
            const float d = (i < q) ? dtg[(long long)i * H] : 0.f;
            vDt[i] = d;
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
        for (int k = 0; k < R; ++k) vS2[lane * R + k] = (excl + a[k]) * kLog2e;
    }
    // stage B rows while wave 0 scans
#pragma unroll
    for (int k = 0; k < NVB; ++k) {
        const int v = tid + k * S::kThreads;
        const int j = v / VPR;
        const int c = v - j * VPR;
        if (v < Q * VPR) *reinterpret_cast<i32x4 *>(sB + j * S::SB + c * (16 / S::E)) = bval[k];
    }
    // stage x transposed: x^T[p][i .. i+3] from 4 tokens of one channel
#pragma unroll
    for (int k = 0; k < NU; ++k) {
        const int u = tid + k * S::kThreads;
        if (u < NUNIT) {
            const int it = u / PB;
            const int p0 = (u - it * PB) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                Half v;
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = xr[k][t][e];
                *reinterpret_cast<Half *>(sX + (p0 + e) * S::SX + 4 * it) = v;
            }
        }
    }
    __syncthreads();
    const float s2_last = vS2[Q - 1];
    for (int i = tid; i < Q; i += S::kThreads) {
        const float s2 = vS2[i];
        const float d = vDt[i];
        const float ref = vS2[i | 15];
        vCol[i] = exp2f_fast(ref - s2) * d;
        vW[i] = exp2f_fast(s2_last - s2) * d;
        vEo[i] = exp2f_fast(s2);
        if ((i & 15) == 15) vRef[i >> 4] = s2;
    }
    if constexpr (S::NP != N) {
        for (int v = tid; v < P * (S::NP - N); v += S::kThreads) {
            const int p = v / (S::NP - N);
            sH[p * S::SH + N + (v - p * (S::NP - N))] = from_f32<IO>(0.f);
        }
    }
    __syncthreads();

    // ---- chunk state, transposed: S_c^T = (B^T o w) x : N x P, K = chunk ----
    // Accumulator element r of tile (nt, pt) is S_c[p][n] with
    // p = pt*16 + li and n = nt*16 + 4*lg + r (four consecutive state columns).
    const int wn = wave % S::WN;
    const int wp = wave / S::WN;
    f32x4 accS[S::NTW][S::PTW];
#pragma unroll
    for (int a = 0; a < S::NTW; ++a)
#pragma unroll
        for (int b = 0; b < S::PTW; ++b) accS[a][b] = zero4();
    if (wp < S::PT) {
#pragma unroll 2
        for (int ks = 0; ks < S::QK; ++ks) {
            const f32x4 wlo = *reinterpret_cast<const f32x4 *>(vW + ks * 32 + 8 * lg);
            const f32x4 whi = *reinterpret_cast<const f32x4 *>(vW + ks * 32 + 8 * lg + 4);
            Frag xf[S::PTW];
#pragma unroll
            for (int b = 0; b < S::PTW; ++b) {
                const int pt = wp + b * S::WP;
                xf[b] = zero_frag<Frag>();
                if (pt < S::PT)
                    xf[b] = *reinterpret_cast<const Frag *>(sX + (pt * 16 + li) * S::SX + ks * 32 + 8 * lg);
            }
#pragma unroll
            for (int a = 0; a < S::NTW; ++a) {
                const int nt = wn + a * S::WN;
                if (nt < S::NT) {
                    const Frag bt = scale_frag<IO>(load_bt_frag<IO, S::SB>(sB, ks * 32, nt * 16, li, lg), wlo, whi);
#pragma unroll
                    for (int b = 0; b < S::PTW; ++b) {
                        const int pt = wp + b * S::WP;
                        if (pt < S::PT) accS[a][b] = Io<IO>::mfma(accS[a][b], bt, xf[b]);
                    }
                }
            }
        }
    }

    // ---- wait for the incoming boundary state, publish the outgoing one ----
    // The boundary state and the progress flag are accessed with device-scope
    // coherent operations (sc1): stores write through to the device coherence
    // point and loads read from it, so no L2 write-back or invalidate is
    // needed.  The producer waits until its state stores are acknowledged
    // before the flag store; the consumer polls the flag and only then loads.
    const int unit = seq * H + h;
    if (cloc > 0) {
        if (tid == 0) {
            int it = 0;
            while (__hip_atomic_load(prm.flags + unit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < cloc) {
                __builtin_amdgcn_s_sleep(1);
                if (++it > (1 << 22)) {
                    atomicOr(prm.error, 1);
                    break;
                }
            }
        }
        __syncthreads();
    }
    const float *hin = (cloc == 0) ? (prm.init_state ? prm.init_state + (long long)unit * P * N : nullptr)
                                   : prm.state + (long long)unit * P * N;
    float *hout = prm.state + (long long)unit * P * N;
    const float alpha = exp2f_fast(s2_last);
    if (wp < S::PT) {
        constexpr int kDevice = 16;  // cache policy: sc1 (device scope)
        const __amdgpu_buffer_rsrc_t rin =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(hin), 0, hin ? P * N * 4 : 0, 0x00020000);
        const __amdgpu_buffer_rsrc_t rout = __builtin_amdgcn_make_buffer_rsrc(hout, 0, P * N * 4, 0x00020000);
        f32x4 hv[S::NTW][S::PTW];
#pragma unroll
        for (int a = 0; a < S::NTW; ++a)
#pragma unroll
            for (int b = 0; b < S::PTW; ++b) {
                const int nt = wn + a * S::WN, pt = wp + b * S::WP;
                hv[a][b] = zero4();
                if (nt < S::NT && pt < S::PT && hin)
                    hv[a][b] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                        rin, ((pt * 16 + li) * N + nt * 16 + 4 * lg) * 4, 0, kDevice));
            }
#pragma unroll
        for (int a = 0; a < S::NTW; ++a)
#pragma unroll
            for (int b = 0; b < S::PTW; ++b) {
                const int nt = wn + a * S::WN, pt = wp + b * S::WP;
                if (nt < S::NT && pt < S::PT) {
                    const int p = pt * 16 + li;
                    const int n0 = nt * 16 + 4 * lg;
                    f32x4 o;
                    Half hb;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        o[r] = alpha * hv[a][b][r] + accS[a][b][r];
                        hb[r] = from_f32<IO>(hv[a][b][r]);
                    }
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, o), rout, (p * N + n0) * 4, 0,
                                                           kDevice);
                    *reinterpret_cast<Half *>(sH + p * S::SH + n0) = hb;
                }
            }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's state stores are acknowledged
    __syncthreads();
    if (tid == 0) __hip_atomic_store(prm.flags + unit, cloc + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // ---- outputs, one 16-row tile at a time ----
#pragma unroll 1
    for (int k = 0;; ++k) {
        const int I = snake_tile(wave, k, S::kWaves);
        if (I >= S::QT) break;
        const int i0 = I * 16;
        if (i0 >= q) continue;
        // C rows as fragments (B operand of B C^T, A operand of C H^T)
        Frag cf[S::NK];
        {
            const int i = i0 + li;
#pragma unroll
            for (int ks = 0; ks < S::NK; ++ks) {
                const int n0 = ks * 32 + 8 * lg;
                cf[ks] = zero_frag<Frag>();
                if (i < q && n0 < N) cf[ks] = *reinterpret_cast<const Frag *>(Cg + i * bs + n0);
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
        // diagonal block: (C B^T o Lambda) diag(dt) x, 32 columns per step
        const int i_row = i0 + li;
        const float s2_i = vS2[i_row];
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
            // lane holds G[i_row][j] for j = 32 kj + 16 half + 4 lg + r
            Frag m;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int jt = 2 * kj + half;
                const int j0 = 32 * kj + 16 * half + 4 * lg;
                if (jt < I) {
                    const float rowf = exp2f_fast(s2_i - vRef[jt]);
                    const f32x4 col = *reinterpret_cast<const f32x4 *>(vCol + j0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) m[4 * half + r] = from_f32<IO>(gt[half][r] * rowf * col[r]);
                } else if (jt == I) {
                    const f32x4 s2j = *reinterpret_cast<const f32x4 *>(vS2 + j0);
                    const f32x4 dtj = *reinterpret_cast<const f32x4 *>(vDt + j0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float v = gt[half][r] * exp2f_fast(s2_i - s2j[r]) * dtj[r];
                        m[4 * half + r] = from_f32<IO>((j0 + r <= i_row) ? v : 0.f);
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) m[4 * half + r] = from_f32<IO>(0.f);
                }
            }
#pragma unroll
            for (int pt = 0; pt < S::PT; ++pt) {
                const IO *xrp = sX + (pt * 16 + li) * S::SX + 32 * kj + 4 * lg;
                const Half lo = *reinterpret_cast<const Half *>(xrp);
                const Half hi = *reinterpret_cast<const Half *>(xrp + 16);
                const Frag xf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                accY[pt] = Io<IO>::mfma(accY[pt], m, xf);
            }
        }
        // y = Y_diag + exp(s_i) Y_off + D x, rows i0 + 4 lg + r
        const f32x4 eo = *reinterpret_cast<const f32x4 *>(vEo + i0 + 4 * lg);
#pragma unroll
        for (int pt = 0; pt < S::PT; ++pt) {
            const Half xv = *reinterpret_cast<const Half *>(sX + (pt * 16 + li) * S::SX + i0 + 4 * lg);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = i0 + 4 * lg + r;
                if (i < q) {
                    const float yv = accY[pt][r] + eo[r] * accO[pt][r] + Dh * to_f32(xv[r]);
                    yg[i * xs + pt * 16 + li] = from_f32<IO>(yv);
                }
            }
        }
    }
}

}  // namespace ssd

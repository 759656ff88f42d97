// ssd_fwd_kernel.h -- fused chunked SSD forward kernel for gfx950.
//
// Algorithm ("Transformers are SSMs Review", section 3-2(4): split the
// sequence into chunks, evaluate the diagonal blocks in the quadratic masked
// form, carry chunk-boundary states between chunks, fold them back into the
// outputs).  Per (sequence, head h, chunk c) with in-chunk index i in [0, q),
// a_t = dt_t A_h and s_i the inclusive in-chunk cumulative sum of a:
//   G       = C B^T                                      (per chunk and group)
//   Y_diag  = (G o Lambda) diag(dt) X,   Lambda_ij = exp(s_i - s_j), j <= i
//   S_c     = X^T diag(exp(s_{q-1} - s_j) dt_j) B        (chunk state from 0)
//   H_{c+1} = exp(s_{q-1}) H_c + S_c                     (inter-chunk recurrence)
//   Y_off   = diag(exp(s_i)) C H_c^T
//   y       = Y_diag + Y_off + D_h x
//
// Work decomposition.  A workgroup (8 waves) owns one chunk of one B/C group
// and a slice of that group's heads.  C B^T depends only on the chunk and the
// group (heads of a group share B and C: the multi-input head pattern of
// section 3-2(5)), so it is formed once per workgroup and kept in registers:
// wave w owns the 16-row tiles w and 15 - w of the chunk (balanced causal
// work) and holds their lower-triangular C B^T tiles.  B stays in LDS and the
// wave's C rows stay in registers while the workgroup walks over its heads;
// per head only x and dt are loaded (prefetched during the previous head).
//
// Chain.  Work items (chunk entry, group, head slice) are listed per XCD:
// all chunks of one (sequence, group, slice) chain belong to the same XCD, and
// each list is in chunk-index-major order.  A workgroup reads its XCD id and
// takes tickets from that XCD's counter until the list is exhausted, so the
// workgroup holding chunk c-1 of a chain took its ticket earlier and walks the
// heads in the same order: the chain cannot deadlock.  For each head the
// workgroup forms S_c and the diagonal blocks, then waits for the
// predecessor's boundary state (a counter per (sequence, head) that each of
// the predecessor's waves increments once its part of H_c is stored), updates
// it and hands H_{c+1} on.  Producer and consumer share the XCD's L2, so the
// state moves with ordinary stores and L1-bypassing loads.  The state buffer
// is the caller's final_state (or workspace); it ends up holding the final
// state.
//
// Numerics.  All decays are products of factors <= 1 (A <= 0, dt >= 0):
// for a 16 x 16 tile (I, J) below the diagonal,
//   exp(s_i - s_j) = exp(s_i - s_r) * exp(s_r - s_j),  r = last token of tile J,
// so only the diagonal tiles need a per-element exponential; the chunk-state
// weights exp(s_{q-1} - s_j) and the read-out weights exp(s_i) are per-token
// vectors.  Exponentials are evaluated as exp2 of log2(e)-scaled sums.
// Accumulation and the boundary state are fp32.
#pragma once

#include <climits>
#include <type_traits>

#include "ssd_device.h"

namespace ssd {

struct FwdParams {
    const void *x;
    const float *dt;
    DtProc dtp;               // optional step-size preprocessing
    const float *A;
    const void *B;
    const void *C;
    const float *D;           // may be null
    const float *init_state;  // may be null
    void *y;
    float *state;             // boundary-state buffer; holds the final state at the end
    const int4 *chunks;       // {seq, chunk index in seq, first token, length}
    const int *n_chunks;      // number of valid chunk entries
    int *tickets;             // one counter per XCD
    const int *items;         // per-XCD work-item lists, concatenated
    const int *xcd_count;     // items per XCD
    const int *xcd_offset;    // start of each XCD's list
    int n_xcd;
    int *flags;               // per (sequence, head): published state parts (kWaves per chunk)
    int *error;
    int H, G;
    int heads_per_item;       // head slice length (the last slice of a group may be shorter)
    int slices;               // slices per group: ceil((H / G) / heads_per_item)
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
    static constexpr int QT = Q / 16;            // 16-row tiles of a chunk (<= 2 per wave)
    static constexpr int QK = Q / 32;            // K steps over a chunk
    static constexpr bool kTwoTiles = QT > kWaves;   // waves own tiles w and 2*kWaves-1-w
    static constexpr int GT = kTwoTiles ? QT + 1 : QT; // C B^T tiles held per wave
    // chunk-state work split: WN waves along the state dim, WP along the head dim
    static constexpr int WN = cmin(NT, kWaves);
    static constexpr int WP = kWaves / WN;
    static constexpr int NTW = (NT + WN - 1) / WN;   // state tiles per wave
    static constexpr int PTW = (PT + WP - 1) / WP;   // head-dim tiles per wave
    static constexpr int E = (int)sizeof(IO);
    static constexpr int PAD = 16 / E;           // 16 bytes of padding per LDS row
    static constexpr int SB = NP + PAD;          // row stride of the B chunk
    static constexpr int SX = Q + PAD;           // row stride of the x^T tile
    static constexpr int SH = NP + PAD;          // row stride of the incoming state
    static constexpr int kLdsB = Q * SB * E;
    static constexpr int kLdsX = P * SX * E;
    static constexpr int kLdsH = P * SH * E;
    static constexpr int kNVec = 7;              // per-token float vectors (+ dt/A staging)
    static constexpr int kLdsVec = kNVec * Q * 4 + 16;
    static constexpr int kLds = kLdsB + kLdsX + kLdsH + kLdsVec + 16;
    static constexpr bool kFits = kLds <= 160 * 1024 && QT <= 2 * kWaves;
};

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2f_fast(float v) { return __builtin_amdgcn_exp2f(v); }

// v + (value of v in the lane selected by the DPP control `ctrl`), where lanes
// without a source (or outside `row_mask`) add 0.
template <int ctrl, int row_mask>
__device__ __forceinline__ float dpp_add(float v) {
    const int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, row_mask, 0xF, true);
    return v + __builtin_bit_cast(float, t);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: four
// shifts inside each 16-lane row, then row 0 and 2's last lane into rows 1
// and 3, then lane 31 into rows 2 and 3.
__device__ __forceinline__ float wave_inclusive_sum(float v) {
    v = dpp_add<0x111, 0xF>(v);   // row_shr:1
    v = dpp_add<0x112, 0xF>(v);   // row_shr:2
    v = dpp_add<0x114, 0xF>(v);   // row_shr:4
    v = dpp_add<0x118, 0xF>(v);   // row_shr:8
    v = dpp_add<0x142, 0xA>(v);   // row_bcast:15
    v = dpp_add<0x143, 0xC>(v);   // row_bcast:31
    return v;
}

// K-slot order.  Every contraction over chunk tokens uses the same slot
// order: within a 32-token K step, slot e (0..7) of lane group lg holds token
//     16 * (e / 4) + 4 * lg + e % 4,
// which is the row order of the 16 x 16 C B^T accumulator tiles (two tiles
// side by side).  The staged x^T stores tokens at the matching permuted
// position (8 * lg + e within each 32-token block), so every x operand is one
// contiguous 16-byte LDS read.
__device__ __forceinline__ int xpos(int j) {
    return (j & ~31) | (((j >> 2) & 3) << 3) | (((j >> 4) & 1) << 2) | (j & 3);
}

// Unscaled B^T fragment in the K-slot order above: lane holds
// B[k0 + 16 * (e / 4) + 4 * lg + e % 4][n0 + li], e = 0..7.
template <typename IO, int SB>
__device__ __forceinline__ typename Io<IO>::Frag load_bt_frag(const IO *sB, int k0, int n0, int li, int lg) {
    typename Io<IO>::Frag f;
    if constexpr (sizeof(IO) == 2) {
        const int row = k0 + 4 * lg + (li >> 2);
        const int col = n0 + 4 * (li & 3);
        const bf16x4 lo = lds_read_tr16(reinterpret_cast<const bf16 *>(sB + row * SB + col));
        const bf16x4 hi = lds_read_tr16(reinterpret_cast<const bf16 *>(sB + (row + 16) * SB + col));
        f = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = sB[(k0 + 16 * (e >> 2) + 4 * lg + (e & 3)) * SB + n0 + li];
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

// Registers holding one head's x chunk (units of 4 tokens x 8 channels) and,
// in wave 0, its dt (Q/64 consecutive tokens per lane, the layout of the
// in-chunk scan) between their global load and their use.
template <typename IO, int P, int N, int Q>
struct Prefetch {
    typedef FwdShape<IO, P, N, Q> S;
    typedef typename Io<IO>::Frag Frag;
    static constexpr int PB = P / 8;
    static constexpr int NUNIT = (Q / 4) * PB;
    static constexpr int NU = (NUNIT + S::kThreads - 1) / S::kThreads;
    static constexpr int R = Q / 64;
    Frag x[NU][4];
    float dt[R];
    float a;   // A[h] (wave 0)
    float braw; // dt_bias[h] (A[h] when there is no bias; not used then)

    // Unit u covers tokens 4*t4 .. 4*t4+3 and channels p0 .. p0+7.  Sixteen
    // consecutive units take sixteen consecutive token groups of one channel
    // block, so the transposing LDS writes of 16 lanes hit distinct banks.
    static __device__ __forceinline__ int unit_t4(int u) { return (u & 15) + 16 * (u / (16 * PB)); }
    static __device__ __forceinline__ int unit_p0(int u) { return ((u >> 4) % PB) * 8; }

    __device__ __forceinline__ void load(const FwdParams &prm, long long tok0, int q, int h, int tid) {
        const int xs = prm.H * P;
        const IO *xg = reinterpret_cast<const IO *>(prm.x) + tok0 * xs + h * P;
#pragma unroll
        for (int k = 0; k < NU; ++k) {
            const int u = tid + k * S::kThreads;
            const int t4 = unit_t4(u);
            const int p0 = unit_p0(u);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int i = 4 * t4 + t;
                x[k][t] = zero_frag<Frag>();
                if (u < NUNIT && i < q) x[k][t] = *reinterpret_cast<const Frag *>(xg + i * xs + p0);
            }
        }
        if (tid < 64) {
#pragma unroll
            for (int k = 0; k < R; ++k) {
                const int i = tid * R + k;
                dt[k] = (i < q) ? prm.dt[(tok0 + i) * prm.H + h] : 0.f;
            }
            a = prm.A[h];
            braw = (prm.dtp.bias ? prm.dtp.bias : prm.A)[h];   // branch-free
        }
    }

    // wave 0: dt (lane holds tokens R*lane .. R*lane+R-1, preprocessed when
    // asked; tokens past the chunk stay 0) and A into LDS
    __device__ __forceinline__ void stage_dt(float *sStage, int lane, int q, const DtProc &dtp) const {
#pragma unroll
        for (int k = 0; k < R; ++k) {
            float v = dt[k];
            if (dtp.on && lane * R + k < q) v = dtp.apply(v, dtp.bias ? braw : 0.f);
            sStage[lane * R + k] = v;
        }
        if (lane == 0) sStage[Q] = a;
    }

    // x^T[p][i .. i+3] from 4 tokens of one channel
    __device__ __forceinline__ void stage(IO *sX, int tid) const {
        typedef typename Io<IO>::Half Half;
#pragma unroll
        for (int k = 0; k < NU; ++k) {
            const int u = tid + k * S::kThreads;
            if (u < NUNIT) {
                const int t4 = unit_t4(u);
                const int p0 = unit_p0(u);
                const int pos = xpos(4 * t4);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    Half v;
#pragma unroll
                    for (int t = 0; t < 4; ++t) v[t] = x[k][t][e];
                    *reinterpret_cast<Half *>(sX + (p0 + e) * S::SX + pos) = v;
                }
            }
        }
    }
};

template <typename IO, int P, int N, int Q>
__global__ __launch_bounds__(512) void ssd_fwd_kernel(FwdParams prm) {
    typedef FwdShape<IO, P, N, Q> S;
    typedef typename Io<IO>::Frag Frag;
    typedef typename Io<IO>::Half Half;
    static_assert(S::kFits, "chunk tiles do not fit in LDS");

    __shared__ __attribute__((aligned(16))) char smem[S::kLds];
    // The small per-token vectors and the x^T and state tiles come first, so
    // that their addresses fit the 16-bit immediate offset of LDS instructions;
    // the B chunk (the largest tile) is last.
    float *vS2 = reinterpret_cast<float *>(smem);  // s * log2(e)
    IO *sX = reinterpret_cast<IO *>(smem + S::kLdsVec + 16);
    IO *sH = reinterpret_cast<IO *>(smem + S::kLdsVec + 16 + S::kLdsX);
    IO *sB = reinterpret_cast<IO *>(smem + S::kLdsVec + 16 + S::kLdsX + S::kLdsH);
    float *vDt = vS2 + Q;     // dt_j
    float *vCol = vDt + Q;    // exp(s_r - s_j) dt_j, r = last token of j's 16-tile
    float *vW = vCol + Q;     // exp(s_last - s_j) dt_j
    float *vEo = vW + Q;      // exp(s_i)
    float *vRef = vEo + Q;    // s2 of the last token of each 16-tile (QT used)
    float *sStage = vRef + Q; // next head's dt (Q values) and A, staged by wave 0
    int *sTicket = reinterpret_cast<int *>(sStage + Q + 4);

    int tid = threadIdx.x;
    int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(wave >= 0 && wave < S::kWaves);
    int li = lane & 15;
    int lg = lane >> 4;
    const int H = prm.H;
    const int G = prm.G;

    // This workgroup's XCD; it only takes items of that XCD's list, so every
    // chunk of a (sequence, head) chain runs on one XCD and the boundary state
    // passes through that XCD's L2.
    const int xcd = (int)(__builtin_amdgcn_s_getreg((15 << 11) | 20) & 15) % prm.n_xcd;  // HW_REG_XCC_ID
#pragma unroll 1
    for (;;) {
        if (tid == 0) {
            const int t = atomicAdd(prm.tickets + xcd, 1);
            sTicket[0] = t < prm.xcd_count[xcd] ? prm.items[prm.xcd_offset[xcd] + t] : -1;
        }
        __syncthreads();
        const int ticket = sTicket[0];
        if (ticket < 0) break;
        const int per_entry = G * prm.slices;
        const int entry = ticket / per_entry;
        const int rem = ticket - entry * per_entry;
        const int g = rem / prm.slices;
        const int slice = rem - g * prm.slices;
        const int hpg = H / G;
        const int h_begin = g * hpg + slice * prm.heads_per_item;
        const int h_end = min(h_begin + prm.heads_per_item, (g + 1) * hpg);
        const int4 ce = prm.chunks[entry];
        const int seq = ce.x;
        const int cloc = ce.y;
        const long long tok0 = ce.z;
        const int q = ce.w;
        const int xs = H * P;          // token stride of x and y (elements)
        const int bs = G * N;          // token stride of B and C
        const IO *Bg = reinterpret_cast<const IO *>(prm.B) + tok0 * bs + g * N;
        const IO *Cg = reinterpret_cast<const IO *>(prm.C) + tok0 * bs + g * N;

        // ---- first head's x and dt, then the B chunk (row layout) into LDS ----
        Prefetch<IO, P, N, Q> pf;
        pf.load(prm, tok0, q, h_begin, tid);
        {
            constexpr int VPR = S::NP * S::E / 16;   // 16-byte vectors per padded row
            constexpr int VN = N * S::E / 16;        // vectors that hold data
            constexpr int NV = (Q * VPR + S::kThreads - 1) / S::kThreads;
            i32x4 bv[NV];
    #pragma unroll
            for (int k = 0; k < NV; ++k) {
                const int u = tid + k * S::kThreads;
                const int j = u / VPR;
                const int c = u - j * VPR;
                bv[k] = i32x4{0, 0, 0, 0};
                if (u < Q * VPR && j < q && c < VN) bv[k] = *reinterpret_cast<const i32x4 *>(Bg + j * bs + c * (16 / S::E));
            }
    #pragma unroll
            for (int k = 0; k < NV; ++k) {
                const int u = tid + k * S::kThreads;
                const int j = u / VPR;
                const int c = u - j * VPR;
                if (u < Q * VPR) *reinterpret_cast<i32x4 *>(sB + j * S::SB + c * (16 / S::E)) = bv[k];
            }
        }

        // ---- this wave's row tiles, their C rows and their C B^T tiles ----
        // Tile Ia = wave; tile Ib = 2*kWaves-1-wave when the chunk has 2*kWaves
        // tiles.  gtile[J] holds C B^T tile (Ia, J); gtile[GT-1-J] holds (Ib, J).
        const int Ia = wave;
        const int Ib = S::kTwoTiles ? 2 * S::kWaves - 1 - wave : S::QT;
        const bool hasA = Ia < S::QT && 16 * Ia < q;
        const bool hasB = S::kTwoTiles && 16 * Ib < q;
        // C rows of tile I as fragments (B operand of B C^T and of H C^T)
        auto load_c = [&](int I, Frag (&cf)[S::NK]) {
    #pragma unroll
            for (int ks = 0; ks < S::NK; ++ks) {
                const int n0 = ks * 32 + 8 * lg;
                cf[ks] = zero_frag<Frag>();
                if (16 * I + li < q && n0 < N) cf[ks] = *reinterpret_cast<const Frag *>(Cg + (16 * I + li) * bs + n0);
            }
        };
        Frag cga[S::NK], cgb[S::NK];
        load_c(hasA ? Ia : S::QT, cga);
        load_c(hasB ? Ib : S::QT, cgb);
        if (wave == 0) pf.stage_dt(sStage, lane, q, prm.dtp);
        __syncthreads();  // B chunk and the first head's dt in LDS
        // Kept in the io precision (the decay-weighted mask built from it is
        // rounded to the io type for the MFMA anyway); fp32 accumulation.
        Half gtile[S::GT];
    #pragma unroll
        for (int J = 0; J < S::GT; ++J) {
            // (Ia, J) for J <= Ia, else (Ib, GT-1-J) for GT-1-J <= Ib
    #pragma unroll
            for (int r = 0; r < 4; ++r) gtile[J][r] = from_f32<IO>(0.f);
            const bool useA = J <= Ia;
            const int jt = useA ? J : S::GT - 1 - J;
            const bool live = useA ? hasA : (hasB && jt <= Ib);
            if (live) {
                f32x4 acc = zero4();
    #pragma unroll
                for (int ks = 0; ks < S::NK; ++ks) {
                    const Frag bfr = *reinterpret_cast<const Frag *>(sB + (16 * jt + li) * S::SB + ks * 32 + 8 * lg);
                    acc = Io<IO>::mfma(acc, bfr, useA ? cga[ks] : cgb[ks]);
                }
    #pragma unroll
                for (int r = 0; r < 4; ++r) gtile[J][r] = from_f32<IO>(acc[r]);
            }
        }

        const int wn = wave % S::WN;
        const int wp = wave / S::WN;

        // Diagonal block of tile I (transposed, Y^T = x^T M^T): accumulator
        // element r of tile pt is Y_diag[16 I + li][pt*16 + 4*lg + r].  `fromA`
        // selects which end of gtile holds the tile's C B^T row.  The LDS
        // operands of K step kj+1 are read before step kj's arithmetic (the
        // scheduling barriers keep that order); sref holds the 16-tile
        // reference cumsums in scalar registers.
        auto diag_block = [&](auto from_a, int I, f32x4 (&accY)[S::PT], const float (&sref)[S::QT]) {
            constexpr bool fromA = decltype(from_a)::value;
            const int i_row = 16 * I + li;
            const float s2_i = vS2[i_row];
    #pragma unroll
            for (int pt = 0; pt < S::PT; ++pt) accY[pt] = zero4();
            Frag xf[2][S::PT];
            f32x4 colv[2][2];
            auto load_step = [&](int kj, Frag (&xo)[S::PT], f32x4 (&co)[2]) {
    #pragma unroll
                for (int pt = 0; pt < S::PT; ++pt)
                    xo[pt] = *reinterpret_cast<const Frag *>(sX + (pt * 16 + li) * S::SX + 32 * kj + 8 * lg);
    #pragma unroll
                for (int half = 0; half < 2; ++half)
                    co[half] = *reinterpret_cast<const f32x4 *>(vCol + 32 * kj + 16 * half + 4 * lg);
            };
            load_step(0, xf[0], colv[0]);
    #pragma unroll
            for (int kj = 0; kj < S::QT / 2; ++kj) {
                if (kj > I / 2) break;
                const int cur = kj & 1;
                if (kj + 1 < S::QT / 2 && kj + 1 <= I / 2) load_step(kj + 1, xf[cur ^ 1], colv[cur ^ 1]);
                __builtin_amdgcn_sched_barrier(0);
                Frag m;  // lane holds M[i_row][j], j = 32 kj + 16 half + 4 lg + r
    #pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int jt = 2 * kj + half;
                    const int j0 = 32 * kj + 16 * half + 4 * lg;
                    const Half &gh = gtile[fromA ? jt : S::GT - 1 - jt];   // C B^T tile (I, jt)
                    f32x4 gv;
    #pragma unroll
                    for (int r = 0; r < 4; ++r) gv[r] = to_f32(gh[r]);
                    if (jt < I) {
                        const float rowf = exp2f_fast(s2_i - sref[jt]);
    #pragma unroll
                        for (int r = 0; r < 4; ++r) m[4 * half + r] = from_f32<IO>(gv[r] * rowf * colv[cur][half][r]);
                    } else if (jt == I) {
                        const f32x4 s2j = *reinterpret_cast<const f32x4 *>(vS2 + j0);
                        const f32x4 dtj = *reinterpret_cast<const f32x4 *>(vDt + j0);
    #pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float v = gv[r] * exp2f_fast(s2_i - s2j[r]) * dtj[r];
                            m[4 * half + r] = from_f32<IO>((j0 + r <= i_row) ? v : 0.f);
                        }
                    } else {
    #pragma unroll
                        for (int r = 0; r < 4; ++r) m[4 * half + r] = from_f32<IO>(0.f);
                    }
                }
    #pragma unroll
                for (int pt = 0; pt < S::PT; ++pt) accY[pt] = Io<IO>::mfma(accY[pt], xf[cur][pt], m);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // State read-out (H C^T) and the final combination of tile I.
        auto finish_tile = [&](int I, const Frag (&cf)[S::NK], const f32x4 (&accY)[S::PT], IO *yg, float Dh) {
            const int i_row = 16 * I + li;
            f32x4 accO[S::PT];
    #pragma unroll
            for (int pt = 0; pt < S::PT; ++pt) accO[pt] = zero4();
            // software pipeline: the H fragments of K step ks+1 are read while the
            // MFMAs of step ks run (the scheduling barriers keep that order)
            Frag hf[2][S::PT];
            auto load_h = [&](int ks, Frag (&o)[S::PT]) {
    #pragma unroll
                for (int pt = 0; pt < S::PT; ++pt)
                    o[pt] = *reinterpret_cast<const Frag *>(sH + (pt * 16 + li) * S::SH + ks * 32 + 8 * lg);
            };
            load_h(0, hf[0]);
    #pragma unroll
            for (int ks = 0; ks < S::NK; ++ks) {
                if (ks + 1 < S::NK) load_h(ks + 1, hf[(ks + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                for (int pt = 0; pt < S::PT; ++pt) accO[pt] = Io<IO>::mfma(accO[pt], hf[ks & 1][pt], cf[ks]);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (i_row < q) {
                const float eo = vEo[i_row];
                float xv[S::PT][4];   // x[i_row][pt*16 + 4 lg + r], all read before use
                const int xp = xpos(i_row);
    #pragma unroll
                for (int pt = 0; pt < S::PT; ++pt)
    #pragma unroll
                    for (int r = 0; r < 4; ++r) xv[pt][r] = to_f32(sX[(pt * 16 + 4 * lg + r) * S::SX + xp]);
                __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                for (int pt = 0; pt < S::PT; ++pt) {
                    Half yv;
    #pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float xval = xv[pt][r];
                        yv[r] = from_f32<IO>(accY[pt][r] + eo * accO[pt][r] + Dh * xval);
                    }
                    *reinterpret_cast<Half *>(yg + i_row * xs + pt * 16 + 4 * lg) = yv;
                }
            }
        };

        int *sReady = sTicket + 1;

    #pragma unroll 1
        for (int h = h_begin; h < h_end; ++h) {
            // Lane indices are made opaque per head so that per-head addresses
            // and predicates are recomputed rather than kept live across heads.
            asm volatile("" : "+v"(tid), "+v"(lane), "+v"(li), "+v"(lg));
            // (and so are the stored C B^T tiles, so that their conversion to
            // fp32 is done at use instead of being hoisted out of the loop)
    #pragma unroll
            for (int J = 0; J < S::GT; ++J) {
                if constexpr (sizeof(IO) == 2) {
                    long long gbits = __builtin_bit_cast(long long, gtile[J]);
                    asm volatile("" : "+v"(gbits));
                    gtile[J] = __builtin_bit_cast(Half, gbits);
                }
            }
            IO *yg = reinterpret_cast<IO *>(prm.y) + tok0 * xs + h * P;
            const int unit = seq * H + h;

            // ---- (1) stage x^T; in-chunk cumulative sum and per-token vectors ----
            pf.stage(sX, tid);
            {
                // one early look at the predecessor's flag (the state loads can
                // then be issued before the compute phase)
                // (compared only after the scan, so that the scan does not wait for it)
                int flagv = INT_MAX;
                if (wave == 0 && lane == 0 && cloc > 0)
                    flagv = __hip_atomic_load(prm.flags + unit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                // Every wave scans the whole chunk (R tokens per lane, from the
                // staged dt) and writes the per-token vectors of its own Q/8
                // tokens (lanes 8 wave .. 8 wave + 7).
                constexpr int R = Q / 64;
                const float Ah = sStage[Q];
                float dtv[R];
    #pragma unroll
                for (int k = 0; k < R; ++k) dtv[k] = sStage[lane * R + k];
                float s2[R];
                float run = 0.f;
    #pragma unroll
                for (int k = 0; k < R; ++k) {
                    run += dtv[k] * Ah;
                    s2[k] = run;
                }
                const float excl = wave_inclusive_sum(run) - run;
    #pragma unroll
                for (int k = 0; k < R; ++k) s2[k] = (excl + s2[k]) * kLog2e;
                const float s2_end = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s2[R - 1]), 63));
                // last token of each 16-token tile: index (i | 15), held by lane ((i | 15) / R)
                const int ref_lane = ((lane * R) | 15) / R;
                const float ref = __shfl(s2[R - 1], ref_lane, 64);
                if ((lane >> 3) == wave) {
    #pragma unroll
                    for (int k = 0; k < R; ++k) {
                        const int i = lane * R + k;
                        const float d = dtv[k];
                        vS2[i] = s2[k];
                        vDt[i] = d;
                        vCol[i] = exp2f_fast(ref - s2[k]) * d;
                        vW[i] = exp2f_fast(s2_end - s2[k]) * d;
                        vEo[i] = exp2f_fast(s2[k]);
                        if ((i & 15) == 15) vRef[i >> 4] = s2[k];
                    }
                }
                asm volatile("" : "+v"(flagv));   // keeps the comparison (and its wait) here
                if (wave == 0 && lane == 0) *sReady = flagv >= S::kWaves * cloc;
            }
            if constexpr (S::NP != N) {
                for (int v = tid; v < P * (S::NP - N); v += S::kThreads) {
                    const int p = v / (S::NP - N);
                    sH[p * S::SH + N + (v - p * (S::NP - N))] = from_f32<IO>(0.f);
                }
            }
            __syncthreads();
            const float s2_last = vS2[Q - 1];
            const bool early = *sReady != 0;
            // the next head's x and dt load while this head is computed
            if (h + 1 < h_end) pf.load(prm, tok0, q, h + 1, tid);

            // incoming boundary state, issued now
            // when the predecessor had already published, else after the wait below
            const float *hin = (cloc == 0) ? (prm.init_state ? prm.init_state + (long long)unit * P * N : nullptr)
                                           : prm.state + (long long)unit * P * N;
            float *hout = prm.state + (long long)unit * P * N;
            // Cache policy of the hand-off: the stores are ordinary, so H_{c+1}
            // stays in this XCD's L2 (write-back); the loads are device scope
            // (sc1), which skips the compute unit's L1 (it may hold an older
            // version of these in-place lines) and is served by the same L2.
            constexpr int kStateLoad = 16;   // sc1
            f32x4 hv[S::NTW][S::PTW];
            auto load_state = [&]() {
                const __amdgpu_buffer_rsrc_t rin =
                    __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(hin), 0, hin ? P * N * 4 : 0, 0x00020000);
    #pragma unroll
                for (int a = 0; a < S::NTW; ++a)
    #pragma unroll
                    for (int b = 0; b < S::PTW; ++b) {
                        const int nt = wn + a * S::WN, pt = wp + b * S::WP;
                        hv[a][b] = zero4();
                        if (wp < S::PT && nt < S::NT && pt < S::PT && hin)
                            hv[a][b] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                rin, ((pt * 16 + li) * N + nt * 16 + 4 * lg) * 4, 0, kStateLoad));
                    }
            };
            if (early) load_state();

            // ---- (2) compute: chunk state and both tiles' diagonal blocks ----
            // S_c^T = (B^T o w) x : N x P, K = chunk; accumulator element r of tile
            // (nt, pt) is S_c[p][n] with p = pt*16 + li and n = nt*16 + 4*lg + r.
            f32x4 accS[S::NTW][S::PTW];
    #pragma unroll
            for (int a = 0; a < S::NTW; ++a)
    #pragma unroll
                for (int b = 0; b < S::PTW; ++b) accS[a][b] = zero4();
            auto chunk_state = [&]() {
            if (wp < S::PT) {
                // software pipeline: the operands of K step ks+1 are read while
                // step ks is scaled and multiplied
                struct ScOps {
                    f32x4 wlo, whi;
                    Frag xf[S::PTW];
                    Frag bt[S::NTW];
                };
                auto load_sc = [&](int ks, ScOps &o) {
                    o.wlo = *reinterpret_cast<const f32x4 *>(vW + ks * 32 + 4 * lg);
                    o.whi = *reinterpret_cast<const f32x4 *>(vW + ks * 32 + 16 + 4 * lg);
    #pragma unroll
                    for (int b = 0; b < S::PTW; ++b) {
                        const int pt = wp + b * S::WP;
                        o.xf[b] = zero_frag<Frag>();
                        if (pt < S::PT)
                            o.xf[b] = *reinterpret_cast<const Frag *>(sX + (pt * 16 + li) * S::SX + ks * 32 + 8 * lg);
                    }
    #pragma unroll
                    for (int a = 0; a < S::NTW; ++a) {
                        const int nt = wn + a * S::WN;
                        o.bt[a] = zero_frag<Frag>();
                        if (nt < S::NT) o.bt[a] = load_bt_frag<IO, S::SB>(sB, ks * 32, nt * 16, li, lg);
                    }
                };
                ScOps ops[2];
                load_sc(0, ops[0]);
    #pragma unroll
                for (int ks = 0; ks < S::QK; ++ks) {
                    const int cur = ks & 1;
                    if (ks + 1 < S::QK) load_sc(ks + 1, ops[cur ^ 1]);
                    __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                    for (int a = 0; a < S::NTW; ++a) {
                        const int nt = wn + a * S::WN;
                        if (nt < S::NT) {
                            const Frag bt = scale_frag<IO>(ops[cur].bt[a], ops[cur].wlo, ops[cur].whi);
    #pragma unroll
                            for (int b = 0; b < S::PTW; ++b) {
                                const int pt = wp + b * S::WP;
                                if (pt < S::PT) accS[a][b] = Io<IO>::mfma(accS[a][b], bt, ops[cur].xf[b]);
                            }
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            };
            // The two waves that share a SIMD (w and w + kWaves/2) take the
            // MFMA-dense chunk state and the VALU-dense diagonal blocks in
            // opposite orders, so that one's matrix work overlaps the other's
            // vector work.
            const bool sc_first = wave < S::kWaves / 2;
            if (sc_first) chunk_state();
            f32x4 accYa[S::PT], accYb[S::PT];
            float sref[S::QT];   // 16-tile reference cumsums, wave-uniform
    #pragma unroll
            for (int t = 0; t < S::QT; ++t)
                sref[t] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, vRef[t])));
            if (hasA) diag_block(std::true_type{}, Ia, accYa, sref);
            if (hasB) diag_block(std::false_type{}, Ib, accYb, sref);
            if (!sc_first) chunk_state();

            Frag cfa[S::NK];
            if (hasA) load_c(Ia, cfa);
            // ---- (3) chain: wait if needed, H_{c+1} = exp(s_last) H_c + S_c, H_c to LDS ----
            if (!early) {
                if (tid == 0) {
                    int it = 0;
                    while (__hip_atomic_load(prm.flags + unit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                           S::kWaves * cloc) {
                        __builtin_amdgcn_s_sleep(1);
                        if (++it > (1 << 22)) {
                            atomicOr(prm.error, 1);
                            break;
                        }
                    }
                }
                __syncthreads();
                load_state();
            }
            const float alpha = exp2f_fast(s2_last);
            const float Dh = prm.D ? prm.D[h] : 0.f;   // needed only by the epilogue
            // every load issued so far (state, C rows of tile Ia, D) completes here, on
            // all paths, so the read-out below only waits for what is issued later
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            if (wp < S::PT) {
                const __amdgpu_buffer_rsrc_t rout = __builtin_amdgcn_make_buffer_rsrc(hout, 0, P * N * 4, 0x00020000);
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
                            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, o), rout, (p * N + n0) * 4,
                                                                   0, 0);
                            *reinterpret_cast<Half *>(sH + p * S::SH + n0) = hb;
                        }
                    }
            }
            __syncthreads();  // H_c is in LDS

            // ---- (4) state read-out and outputs of both tiles ----
            // Each wave publishes its part of H_{c+1} (one increment of the
            // (sequence, head) counter) once its state stores are acknowledged;
            // a successor waits for all kWaves increments.
            Frag cfb[S::NK];
            if (hasB) load_c(Ib, cfb);
            if (hasA) finish_tile(Ia, cfa, accYa, yg, Dh);
            __builtin_amdgcn_s_waitcnt(0);  // this wave's state stores are acknowledged
            if (lane == 0) __hip_atomic_fetch_add(prm.flags + unit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (hasB) finish_tile(Ib, cfb, accYb, yg, Dh);
            if (wave == 0 && h + 1 < h_end) pf.stage_dt(sStage, lane, q, prm.dtp);   // the next head's dt and A
            __syncthreads();  // every wave is done with this head's LDS tiles
        }
    }
}

}  // namespace ssd

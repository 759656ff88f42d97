// ssd_bwd_kernels.h -- backward pass of the SSD layer (gfx950 / CDNA4).
//
// The gradient of L = <dy, y> + <dfinal, final_state> through the chunked
// evaluation of the recurrence ("Transformers are SSMs Review", section
// 3-2(4): quadratic masked form inside a chunk, states passed between
// chunks).  The pages print no backward pass; this is reverse-mode
// differentiation of that forward, per chunk of Q tokens with in-chunk
// cumulative decay s (s_i = sum_{t<=i} dt_t A), d_ij = exp(s_i - s_j) for
// i >= j, w_j = exp(s_last - s_j) dt_j, H_c the state before the chunk and
// R_c the gradient of the state after it:
//
//   R_{c-1} = exp(s_last) R_c + dY^T diag(exp(s)) C                  (reverse chain)
//   E  = dY X^T,   M = (C B^T o d) diag(dt),   W = (E o d) diag(dt)
//   dX = M^T dY + diag(w) B R_c^T + D dY
//   dB = W^T C + diag(w) X R_c          (summed over the heads of a group)
//   dC = W B + diag(exp(s)) dY H_c      (likewise)
//   dL/ds_i = sum_j<=i (M o E)_ij - sum_k>=i (M o E)_ki + exp(s_i) (dY H_c)_i . C_i
//             - w_i (X R_c)_i . B_i + [i = last] <R_c, H_{c+1}>
//   dL/da_j = sum_{i>=j} dL/ds_i,   ddt_j = A dL/da_j + sum_i (C B^T o E o d)_ij
//             + exp(s_last - s_j) (X R_c)_j . B_j,   dA = sum_j dt_j dL/da_j,
//   dD = sum dY . X,   dinit = R_{-1}.
//
// <R_c, H_{c+1}> is evaluated as exp(s_last) <R_c, H_c> + sum_j w_j (X R_c)_j . B_j
// (H_{c+1} expanded by one chunk of the recurrence), so that H_{c+1} is not
// read and its chunk-state part is built from the same products as the
// -w_i (X R_c)_i . B_i terms it cancels against.
//
// Kernels: ssd_bwd_prep_kernel (chunk table), ssd_bwd_scan_kernel (forward
// boundary states H_c, or the reverse chain R_c; one workgroup per
// (sequence, head), chunk-sequential), ssd_bwd_chunk_kernel (everything
// else; one workgroup per (chunk, group), looping over the group's heads so
// that dB and dC accumulate in registers without atomics) and
// ssd_bwd_reduce_kernel (dA and dD from per-chunk partials, in a fixed order).
#pragma once

#include <type_traits>

#include "ssd_device.h"

namespace ssd {

constexpr int kBwdQ = 64;         // tokens per chunk of the backward pass

struct BwdParams {
    const void *x, *B, *C, *dy;   // io
    const float *dt, *A, *D;      // D may be null
    const float *init_state;      // [nseq, H, P, N] or null
    const float *dfinal;          // [nseq, H, P, N] or null
    void *dx;                     // io
    float *ddt, *dB, *dC, *dinit; // dinit may be null
    float *dA, *dD;
    // workspace
    const int4 *chunks;           // [n_chunks] {seq, first token, length, chunk index in seq}
    const int *seq_chunk_start;   // [nseq + 1]
    // (each P x N state row-major, or in state_piece_pos's tile order where
    // the bf16 scans write it for the bf16 chunk kernel)
    float *states;                // [n_chunks + nseq][H][P][N]: H_0 .. H_T of every sequence
    float *radj;                  // [n_chunks][H][P][N]: R_c
    float *partA, *partD;         // [n_chunks][H]
    // H counts kernel heads of P channels.  A head dim wider than the
    // kernel's (128 on 64-channel kernels) runs as `hsub` consecutive kernel
    // heads per model head: x, dy, dx and the states then have the layout of
    // H = hsub * nheads heads (each state row depends only on its own channel
    // of x and on the head's shared dt, A, B, C), while dt, A, D, ddt, dA and
    // dD are indexed by the model head h / hsub, and the sub-heads' terms of
    // ddt, dA and dD are added in a fixed order.
    int H, G, nseq;
    int hsub;                     // kernel heads per model head (1 or 2)
};

// Operand accessors return A[m][k] (row m of the A operand) or B[k][n]; one
// 16 x 16 output tile accumulates over K with the 16x16x32 (bf16) or 16x16x4
// (fp32, eight per K step) MFMA.  acc[r] is Out[m0 + 4 lg + r][n0 + li].
// K steps are 32 wide: slots at or past K (K = 16) are zero and never read.
template <typename IO, typename FA, typename FB>
__device__ __forceinline__ f32x4 mma_tile(f32x4 acc, int K, int lg, FA fa, FB fb) {
    typedef typename Io<IO>::Frag Frag;
    for (int k0 = 0; k0 < K; k0 += 32) {
        Frag a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int k = k0 + 8 * lg + e;
            a[e] = from_f32<IO>(k < K ? fa(k) : 0.f);
            b[e] = from_f32<IO>(k < K ? fb(k) : 0.f);
        }
        acc = Io<IO>::mfma(acc, a, b);
    }
    return acc;
}

// v = hi(v) + lo(v), each representable in the io type: two MFMAs with the
// parts of an fp32 operand carry about 16 mantissa bits through bf16 MFMA
// (fp32 io: hi is v itself and no second product is formed).
template <typename IO> __device__ __forceinline__ float split_hi(float v) { return to_f32(from_f32<IO>(v)); }
template <typename IO> __device__ __forceinline__ float split_lo(float v) { return v - split_hi<IO>(v); }

// Sum over the 64 lanes (wave-uniform result), in a fixed order.
__device__ __forceinline__ float bwd_wave_sum(float v) {
    v = row_sum16(v);
    const auto rl = [&](int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l)); };
    return (rl(0) + rl(16)) + (rl(32) + rl(48));
}

// ---------------------------------------------------------------------------
// Chunk table: sequence chunk offsets and one entry per chunk.
struct BwdPrepParams {
    const int *cu_seqlens;   // null: dense batch
    int batch, seqlen, nseq;
    int *seq_chunk_start;    // [nseq + 1]
    int4 *chunks;
};

__global__ __launch_bounds__(256) void ssd_bwd_prep_kernel(BwdPrepParams p) {
    const int tid = threadIdx.x;
    auto seq_len = [&](int s) { return p.cu_seqlens ? p.cu_seqlens[s + 1] - p.cu_seqlens[s] : p.seqlen; };
    auto seq_start = [&](int s) { return p.cu_seqlens ? p.cu_seqlens[s] : s * p.seqlen; };
    if (tid == 0) {
        int acc = 0;
        for (int s = 0; s < p.nseq; ++s) {
            p.seq_chunk_start[s] = acc;
            acc += (seq_len(s) + kBwdQ - 1) / kBwdQ;
        }
        p.seq_chunk_start[p.nseq] = acc;
    }
    __syncthreads();
    for (int s = 0; s < p.nseq; ++s) {
        const int n = (seq_len(s) + kBwdQ - 1) / kBwdQ;
        const int o = p.seq_chunk_start[s];
        for (int c = tid; c < n; c += 256) {
            const int start = seq_start(s) + c * kBwdQ;
            p.chunks[o + c] = make_int4(s, start, min(kBwdQ, seq_len(s) - c * kBwdQ), c);
        }
    }
}

// Rows [t0, t0 + q) of a [tokens, stride] io tensor, columns [col, col + W),
// into a [Q][W] LDS tile (zeros past q), 8 elements per access.
template <typename IO, int W>
__device__ __forceinline__ void stage_rows(IO *dst, const IO *src, long long t0, int q, long long stride,
                                           long long col, int tid) {
    typedef typename Io<IO>::Frag V;   // 8 elements
    constexpr int V8 = W / 8;
    for (int i = tid; i < kBwdQ * V8; i += 256) {
        const int j = i / V8, c8 = (i - j * V8) * 8;
        V v = zero_frag<V>();
        if (j < q) v = *reinterpret_cast<const V *>(src + (t0 + j) * stride + col + c8);
        *reinterpret_cast<V *>(dst + j * W + c8) = v;
    }
}

// Sum over the 256 threads of a workgroup (all threads get the result).
__device__ __forceinline__ float block_sum(float v, float *scratch) {
    const int wave = threadIdx.x >> 6;
    v = bwd_wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[wave] = v;
    __syncthreads();
    return scratch[0] + scratch[1] + scratch[2] + scratch[3];
}

// ---------------------------------------------------------------------------
// Chunk-sequential scan of one (sequence, head).  MODE 0: forward boundary
// states, states[o + s + c] = H_c (H_0 the initial state, H_T the final
// one).  MODE 1: the reverse chain, radj[o + c] = R_c (R_{T-1} = dfinal) and
// dinit = R_{-1}.  Per chunk the contribution sum_j wt_j u_j (outer) v_j is
// formed on MFMA (u, v = x, B and wt = exp(s_last - s) dt in MODE 0; dy, C and
// wt = exp(s) in MODE 1), and the state is scaled by exp(s_last) first.
template <typename IO, int P, int N, int MODE>
__global__ __launch_bounds__(256) void ssd_bwd_scan_kernel(BwdParams p) {
    constexpr int Q = kBwdQ;
    constexpr int PT = P / 16, NT = N / 16, TILES = PT * NT;
    constexpr int TPW = (TILES + 3) / 4;          // state tiles per wave
    __shared__ __attribute__((aligned(16))) IO su[Q * P];
    __shared__ __attribute__((aligned(16))) IO sv[Q * N];
    __shared__ float swt[Q];
    __shared__ float salpha;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int s = blockIdx.x / p.H, h = blockIdx.x - s * p.H;
    const int g = h / (p.H / p.G);
    const int o = p.seq_chunk_start[s];
    const int nc = p.seq_chunk_start[s + 1] - o;
    const long long PN = (long long)P * N;
    const IO *ug = reinterpret_cast<const IO *>(MODE == 0 ? p.x : p.dy);
    const IO *vg = reinterpret_cast<const IO *>(MODE == 0 ? p.B : p.C);
    const float Ah = p.A[h / p.hsub];

    // Wave w holds state tiles t = w + 4 k, (pt, nt) = (t % PT, t / PT):
    // element r of tile k is state[pt*16 + li][nt*16 + 4 lg + r].
    f32x4 st[TPW];
    const float *st0 = MODE == 0 ? p.init_state : p.dfinal;
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
        const int t = wave + 4 * k;
        st[k] = zero4();
        if (t < TILES && st0) {
            const int pp = (t % PT) * 16 + li, nn = (t / PT) * 16 + 4 * lg;
            st[k] = *reinterpret_cast<const f32x4 *>(st0 + ((long long)s * p.H + h) * PN + pp * N + nn);
        }
    }
    auto store_state = [&](float *dst) {
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int t = wave + 4 * k;
            if (t < TILES) {
                const int pp = (t % PT) * 16 + li, nn = (t / PT) * 16 + 4 * lg;
                *reinterpret_cast<f32x4 *>(dst + pp * N + nn) = st[k];
            }
        }
    };
    if (MODE == 0) store_state(p.states + ((long long)(o + s) * p.H + h) * PN);

    for (int step = 0; step < nc; ++step) {
        const int c = MODE == 0 ? step : nc - 1 - step;
        const int4 ce = p.chunks[o + c];
        const long long t0 = ce.y;
        const int q = ce.z;
        stage_rows<IO, P>(su, ug, t0, q, (long long)p.H * P, (long long)h * P, tid);
        stage_rows<IO, N>(sv, vg, t0, q, (long long)p.G * N, (long long)g * N, tid);
        if (wave == 0) {
            const float d = lane < q ? p.dt[(t0 + lane) * (p.H / p.hsub) + h / p.hsub] : 0.f;
            const float sc = wave_inclusive_sum(d * Ah) * kLog2e;   // s * log2(e)
            const float slast = __shfl(sc, 63, 64);
            swt[lane] = MODE == 0 ? __builtin_amdgcn_exp2f(slast - sc) * d : __builtin_amdgcn_exp2f(sc);
            if (lane == 0) salpha = __builtin_amdgcn_exp2f(slast);
        }
        __syncthreads();
        const float alpha = salpha;
        if (MODE == 1) store_state(p.radj + ((long long)(o + c) * p.H + h) * PN);
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int t = wave + 4 * k;
            if (t < TILES) {
                const int pt = t % PT, nt = t / PT;
                // rows of the product are n (A operand v^T scaled by wt), columns p
                // (B operand u): acc[r] = contribution[pt*16 + li][nt*16 + 4 lg + r]
                // (the scaled operand in two parts: these states meet their own
                // contributions again in the backward's cancelling sums)
                f32x4 acc = mma_tile<IO>(zero4(), Q, lg,
                    [&](int j) { return split_hi<IO>(to_f32(sv[j * N + nt * 16 + li]) * swt[j]); },
                    [&](int j) { return to_f32(su[j * P + pt * 16 + li]); });
                if constexpr (sizeof(IO) == 2)
                    acc = mma_tile<IO>(acc, Q, lg,
                        [&](int j) { return split_lo<IO>(to_f32(sv[j * N + nt * 16 + li]) * swt[j]); },
                        [&](int j) { return to_f32(su[j * P + pt * 16 + li]); });
#pragma unroll
                for (int r = 0; r < 4; ++r) st[k][r] = alpha * st[k][r] + acc[r];
            }
        }
        if (MODE == 0) store_state(p.states + ((long long)(o + s + c + 1) * p.H + h) * PN);
        __syncthreads();
    }
    if (MODE == 1 && p.dinit) store_state(p.dinit + ((long long)s * p.H + h) * PN);
}

// ---------------------------------------------------------------------------
// Everything else, per (chunk, group); the group's heads in turn.
template <typename IO, int P, int N>
__global__ __launch_bounds__(256) void ssd_bwd_chunk_kernel(BwdParams p) {
    constexpr int Q = kBwdQ;
    constexpr int NT = N / 16, PT = P / 16;
    __shared__ __attribute__((aligned(16))) IO xs[Q * P];
    __shared__ __attribute__((aligned(16))) IO dys[Q * P];
    __shared__ __attribute__((aligned(16))) IO Bs[Q * N];
    __shared__ __attribute__((aligned(16))) IO Cs[Q * N];
    __shared__ __attribute__((aligned(16))) float Hs[P * N];   // fp32: see the low-rank products below
    __shared__ __attribute__((aligned(16))) float Rs[P * N];
    __shared__ float Gs[Q * Q];
    __shared__ float Es[Q * Q];
    __shared__ float s2[Q], dtv[Q], ew[Q], es[Q];
    __shared__ float rowZ[Q], colZ[Q], offB[Q], offC[Q];
    __shared__ float red[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int ci = blockIdx.x / p.G, g = blockIdx.x - ci * p.G;
    if (ci >= p.seq_chunk_start[p.nseq]) return;   // the grid is sized for the most chunks possible
    const int4 ce = p.chunks[ci];
    const int s = ce.x, c = ce.w, q = ce.z;
    const long long t0 = ce.y;
    const int o = p.seq_chunk_start[s];
    const int H = p.H, hpg = H / p.G;
    const long long PN = (long long)P * N;

    stage_rows<IO, N>(Bs, reinterpret_cast<const IO *>(p.B), t0, q, (long long)p.G * N, (long long)g * N, tid);
    stage_rows<IO, N>(Cs, reinterpret_cast<const IO *>(p.C), t0, q, (long long)p.G * N, (long long)g * N, tid);
    __syncthreads();
    // G = C B^T: wave w computes row band w (tiles (w, jt), jt = 0..3)
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        const f32x4 acc = mma_tile<IO>(zero4(), N, lg,
            [&](int n) { return to_f32(Cs[(wave * 16 + li) * N + n]); },
            [&](int n) { return to_f32(Bs[(jt * 16 + li) * N + n]); });
#pragma unroll
        for (int r = 0; r < 4; ++r) Gs[(wave * 16 + 4 * lg + r) * Q + jt * 16 + li] = acc[r];
    }

    // dB, dC of the group: wave w owns rows w*16 .. w*16+15, all N columns;
    // element r of tile nt is row w*16 + 4 lg + r, column nt*16 + li
    f32x4 dBacc[NT], dCacc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) dBacc[nt] = dCacc[nt] = zero4();
    const int row0 = wave * 16;

    float ddt_sub = 0.f;   // ddt of a model head summed over its kernel heads (wave 0)
    for (int hh = 0; hh < hpg; ++hh) {
        const int h = g * hpg + hh;
        __syncthreads();   // the previous head's tiles are no longer read
        stage_rows<IO, P>(xs, reinterpret_cast<const IO *>(p.x), t0, q, (long long)H * P, (long long)h * P, tid);
        stage_rows<IO, P>(dys, reinterpret_cast<const IO *>(p.dy), t0, q, (long long)H * P, (long long)h * P, tid);
        const float *Hc = p.states + ((long long)(o + s + c) * H + h) * PN;
        const float *Rc = p.radj + ((long long)(o + c) * H + h) * PN;
        float hrd = 0.f;   // <R_c, H_c>
        for (int i = tid; i < P * N; i += 256) {
            const float hv = Hc[i], rv = Rc[i];
            Hs[i] = hv;
            Rs[i] = rv;
            hrd += hv * rv;
        }
        const float Ah = p.A[h / p.hsub];
        if (wave == 0) {
            const float d = lane < q ? p.dt[(t0 + lane) * (H / p.hsub) + h / p.hsub] : 0.f;
            const float sc = wave_inclusive_sum(d * Ah) * kLog2e;
            const float slast = __shfl(sc, 63, 64);
            s2[lane] = sc;
            dtv[lane] = d;
            ew[lane] = __builtin_amdgcn_exp2f(slast - sc);
            es[lane] = __builtin_amdgcn_exp2f(sc);
        }
        hrd = block_sum(hrd, red);   // (its barriers also publish the tiles above)

        // E = dY X^T, row band w
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            const f32x4 acc = mma_tile<IO>(zero4(), P, lg,
                [&](int pp) { return to_f32(dys[(wave * 16 + li) * P + pp]); },
                [&](int pp) { return to_f32(xs[(jt * 16 + li) * P + pp]); });
#pragma unroll
            for (int r = 0; r < 4; ++r) Es[(wave * 16 + 4 * lg + r) * Q + jt * 16 + li] = acc[r];
        }
        float dd = 0.f;   // dy . x over the chunk
        for (int i = tid; i < Q * P; i += 256) dd += to_f32(dys[i]) * to_f32(xs[i]);
        dd = block_sum(dd, red);
        if (tid == 0) p.partD[(long long)ci * H + h] = dd;

        // row sums of (C B^T o E o d) dt and column sums of (C B^T o E o d)
        {
            const int a = tid >> 2, b0 = (tid & 3) * 16;
            float rz = 0.f, cz = 0.f;
#pragma unroll 4
            for (int u = 0; u < 16; ++u) {
                const int j = b0 + u;   // row a, column j
                if (j <= a) {
                    const float z = Gs[a * Q + j] * Es[a * Q + j] * __builtin_amdgcn_exp2f(s2[a] - s2[j]);
                    rz += z * dtv[j];
                }
                const int i = b0 + u;   // column a, row i
                if (i >= a) cz += Gs[i * Q + a] * Es[i * Q + a] * __builtin_amdgcn_exp2f(s2[i] - s2[a]);
            }
            rz += __shfl_xor(rz, 1, 64);
            rz += __shfl_xor(rz, 2, 64);
            cz += __shfl_xor(cz, 1, 64);
            cz += __shfl_xor(cz, 2, 64);
            if ((tid & 3) == 0) {
                rowZ[a] = rz;
                colZ[a] = cz;
            }
        }

        // dx = M^T dY + diag(w) B R^T + D dY, row band w
        const float Dh = p.D ? p.D[h / p.hsub] : 0.f;
        IO *dxg = reinterpret_cast<IO *>(p.dx);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            f32x4 acc = mma_tile<IO>(zero4(), Q, lg,
                [&](int i) {
                    const int j = row0 + li;
                    return i >= j ? Gs[i * Q + j] * __builtin_amdgcn_exp2f(s2[i] - s2[j]) * dtv[j] : 0.f;
                },
                [&](int i) { return to_f32(dys[i * P + pt * 16 + li]); });
            acc = mma_tile<IO>(acc, N, lg,
                [&](int n) {
                    const int j = row0 + li;
                    return to_f32(Bs[j * N + n]) * ew[j] * dtv[j];
                },
                [&](int n) { return Rs[(pt * 16 + li) * N + n]; });
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = row0 + 4 * lg + r, pp = pt * 16 + li;
                if (j < q)
                    dxg[((t0 + j) * H + h) * P + pp] = from_f32<IO>(acc[r] + Dh * to_f32(dys[j * P + pp]));
            }
        }

        // dB, dC of this head, and the row dot products their low-rank parts feed
        float ob[4] = {0.f, 0.f, 0.f, 0.f}, oc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            // diagonal part of dB: sum_i W[i][j] C[i][n]
            const f32x4 db = mma_tile<IO>(zero4(), Q, lg,
                [&](int i) {
                    const int j = row0 + li;
                    return i >= j ? Es[i * Q + j] * __builtin_amdgcn_exp2f(s2[i] - s2[j]) * dtv[j] : 0.f;
                },
                [&](int i) { return to_f32(Cs[i * N + nt * 16 + li]); });
            // exp(s_last - s_j) (X R)[j][n].  The sums of these products over a
            // chunk cancel against <R_c, H_{c+1}> in dL/ds, so they are formed
            // with R in two parts and scaled in fp32 afterwards.
            f32x4 xb = mma_tile<IO>(zero4(), P, lg,
                [&](int pp) { return to_f32(xs[(row0 + li) * P + pp]); },
                [&](int pp) { return split_hi<IO>(Rs[pp * N + nt * 16 + li]); });
            if constexpr (sizeof(IO) == 2)
                xb = mma_tile<IO>(xb, P, lg,
                    [&](int pp) { return to_f32(xs[(row0 + li) * P + pp]); },
                    [&](int pp) { return split_lo<IO>(Rs[pp * N + nt * 16 + li]); });
#pragma unroll
            for (int r = 0; r < 4; ++r) xb[r] *= ew[row0 + 4 * lg + r];
            // diagonal part of dC: sum_j W[i][j] B[j][n]
            const f32x4 dc = mma_tile<IO>(zero4(), Q, lg,
                [&](int j) {
                    const int i = row0 + li;
                    return j <= i ? Es[i * Q + j] * __builtin_amdgcn_exp2f(s2[i] - s2[j]) * dtv[j] : 0.f;
                },
                [&](int j) { return to_f32(Bs[j * N + nt * 16 + li]); });
            // exp(s_i) (dY H)[i][n], likewise in two parts
            f32x4 yc = mma_tile<IO>(zero4(), P, lg,
                [&](int pp) { return to_f32(dys[(row0 + li) * P + pp]); },
                [&](int pp) { return split_hi<IO>(Hs[pp * N + nt * 16 + li]); });
            if constexpr (sizeof(IO) == 2)
                yc = mma_tile<IO>(yc, P, lg,
                    [&](int pp) { return to_f32(dys[(row0 + li) * P + pp]); },
                    [&](int pp) { return split_lo<IO>(Hs[pp * N + nt * 16 + li]); });
#pragma unroll
            for (int r = 0; r < 4; ++r) yc[r] *= es[row0 + 4 * lg + r];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rr = row0 + 4 * lg + r, nn = nt * 16 + li;
                dBacc[nt][r] += db[r] + dtv[rr] * xb[r];
                dCacc[nt][r] += dc[r] + yc[r];
                ob[r] += xb[r] * to_f32(Bs[rr * N + nn]);
                oc[r] += yc[r] * to_f32(Cs[rr * N + nn]);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int m = 1; m < 16; m <<= 1) {
                ob[r] += __shfl_xor(ob[r], m, 64);
                oc[r] += __shfl_xor(oc[r], m, 64);
            }
            if (li == 0) {
                offB[row0 + 4 * lg + r] = ob[r];
                offC[row0 + 4 * lg + r] = oc[r];
            }
        }
        __syncthreads();

        // ds, its reverse cumulative sum, ddt and the dA partial (wave 0, one token per lane)
        if (wave == 0) {
            const int j = lane;
            const float d = dtv[j];
            // <R_c, H_{c+1}> = exp(s_last) <R_c, H_c> + <R_c, S_c>, and <R_c, S_c> = sum_j dt_j offB_j
            const float rh = __builtin_amdgcn_exp2f(s2[Q - 1]) * hrd + bwd_wave_sum(d * offB[j]);
            float ds = rowZ[j] - d * colZ[j] + offC[j] - d * offB[j] + (j == q - 1 ? rh : 0.f);
            const float tot = bwd_wave_sum(ds);
            const float da = tot - wave_inclusive_sum(ds) + ds;    // sum over i >= j
            const float v = Ah * da + colZ[j] + offB[j];
            ddt_sub = (h % p.hsub == 0) ? v : ddt_sub + v;   // the model head's sub-heads, in order
            if (j < q && h % p.hsub == p.hsub - 1) p.ddt[(t0 + j) * (H / p.hsub) + h / p.hsub] = ddt_sub;
            const float pa = bwd_wave_sum(d * da);
            if (lane == 0) p.partA[(long long)ci * H + h] = pa;
        }
    }

    // dB, dC rows of this chunk for group g
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rr = row0 + 4 * lg + r, nn = nt * 16 + li;
            if (rr < q) {
                p.dB[((t0 + rr) * p.G + g) * N + nn] = dBacc[nt][r];
                p.dC[((t0 + rr) * p.G + g) * N + nn] = dCacc[nt][r];
            }
        }
}

// ---------------------------------------------------------------------------
// bf16 version of the chunk kernel for headdim and dstate >= 32: every MFMA
// operand is read from LDS in the K-slot order of the forward kernel (slot e
// of lane group lg holds k0 + 16 (e / 4) + 4 lg + e % 4): two 8-byte reads for
// an operand whose K index runs along its rows, or two transposing reads when
// it runs down its columns.  C B^T is formed in registers once per chunk; per
// head, dY X^T is formed in registers (a 16-row band per wave), the decayed,
// masked M goes to LDS, W is summed over the heads in registers, and the
// row/column sums of their product come from the same registers.  H and R are
// kept as split bf16 pairs.
template <int S>
__device__ __forceinline__ bf16x8 frag_row(const bf16 *base, int m, int k0, int lg) {
    const bf16 *q = base + m * S + k0 + 4 * lg;
    const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(q);
    const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(q + 16);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int S>
__device__ __forceinline__ bf16x8 frag_col(const bf16 *base, int k0, int n0, int li, int lg) {
    const int row = k0 + 4 * lg + (li >> 2);
    const int col = n0 + 4 * (li & 3);
    const bf16x4 lo = lds_read_tr16(base + row * S + col);
    const bf16x4 hi = lds_read_tr16(base + (row + 16) * S + col);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ f32x4 mfma_bf16(f32x4 acc, bf16x8 a, bf16x8 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

// Order of the chunk states H_c and R_c in the workspace, shared by the
// bf16 scans (writers) and the bf16 chunk kernel (reader): the 16 x 16
// tiles t = pt + (P / 16) nt in turn, each as 64 pieces of 4 floats in the
// lane order of the MFMA accumulator, piece l holding
// state[16 pt + l % 16][16 nt + 4 (l / 16) + 0..3].  A wave's store of one
// tile is then 1 KB of consecutive bytes (in row-major order it is 16 half
// lines).
template <int P>
__device__ __forceinline__ void state_piece_pos(int piece, int &pp, int &nn) {
    constexpr int PT = P / 16;
    const int t = piece >> 6, l = piece & 63;
    pp = (t % PT) * 16 + (l & 15);
    nn = (t / PT) * 16 + 4 * (l >> 4);
}

constexpr int kBwdChunkWaves = 8;   // waves per workgroup of the bf16 chunk kernel (4 or 8)

template <int P, int N, int NW>
__global__ __launch_bounds__(NW * 64) void ssd_bwd_chunk_bf16_kernel(BwdParams p) {
    constexpr int Q = kBwdQ;
    constexpr int NT = N / 16, PT = P / 16;
    constexpr int NTH = NW * 64;                       // threads
    constexpr int NH = NW / 4;                         // column parts: waves w and w + 4 share a row band
    constexpr int NT2 = NT / NH, PT2 = PT / NH;        // tiles per column part
    constexpr int SP = P + 8, SN = N + 8, SQ = Q + 8;   // padded row strides (elements)
    constexpr int XP = Q * P / 8, SP4 = P * N / 4;     // 16-byte x (dy) pieces, 4-float H (R) pieces
    constexpr int XV = (XP + NTH - 1) / NTH, SV = (SP4 + NTH - 1) / NTH;   // per thread, rounded up
    static_assert((NW == 4 || NW == 8) && NT2 >= 1 && PT2 >= 1, "unsupported shape for this kernel");
    __shared__ __attribute__((aligned(16))) bf16 xs[Q * SP];
    __shared__ __attribute__((aligned(16))) bf16 dys[Q * SP];
    __shared__ __attribute__((aligned(16))) bf16 Bs[Q * SN];
    __shared__ __attribute__((aligned(16))) bf16 Cs[Q * SN];
    __shared__ __attribute__((aligned(16))) bf16 Ms[Q * SQ];
    __shared__ __attribute__((aligned(16))) bf16 Ws[Q * SQ];
    __shared__ __attribute__((aligned(16))) bf16 Hh[P * SN];
    __shared__ __attribute__((aligned(16))) bf16 Hl[P * SN];
    __shared__ __attribute__((aligned(16))) bf16 Rh[P * SN];
    __shared__ __attribute__((aligned(16))) bf16 Rl[P * SN];
    __shared__ __attribute__((aligned(16))) bf16 dxs[Q * SP];   // a head's dx rows, written out a head later
    __shared__ float s2[Q], dtv[Q], ew[Q], es[Q];
    __shared__ float rowP[NH][Q], colP[4][Q], offBP[NH][Q], offCP[NH][Q];
    __shared__ float red[NW], hrp[NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int band = wave & 3, half = wave >> 2;
    const int row0 = band * 16;
    const int ci = blockIdx.x / p.G, g = blockIdx.x - ci * p.G;
    if (ci >= p.seq_chunk_start[p.nseq]) return;
    const int4 ce = p.chunks[ci];
    const int s = ce.x, c = ce.w, q = ce.z;
    const long long t0 = ce.y;
    const int o = p.seq_chunk_start[s];
    const int H = p.H, hpg = H / p.G;
    const long long PN = (long long)P * N;
    const bf16 *xg = reinterpret_cast<const bf16 *>(p.x), *dyg = reinterpret_cast<const bf16 *>(p.dy);
    bf16 *dxg = reinterpret_cast<bf16 *>(p.dx);
    // dx rows of head hp from LDS, written as whole rows (P * 2 bytes, in
    // 16-byte pieces; the dx phase's lanes hold 8-byte pieces of 16 tokens)
    auto flush_dx = [&](int hp) {
        for (int i = threadIdx.x; i < Q * (P / 8); i += NTH) {
            const int j = i / (P / 8), c8 = (i % (P / 8)) * 8;
            if (j < q)
                *reinterpret_cast<bf16x8 *>(dxg + ((t0 + j) * H + hp) * P + c8) =
                    *reinterpret_cast<const bf16x8 *>(dxs + j * SP + c8);
        }
    };

    // B and C rows of the chunk (once per group)
    for (int i = tid; i < Q * (N / 8); i += NTH) {
        const int j = i / (N / 8), c8 = (i % (N / 8)) * 8;
        bf16x8 vb = zero_frag<bf16x8>(), vc = zero_frag<bf16x8>();
        if (j < q) {
            vb = *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const bf16 *>(p.B) + ((t0 + j) * p.G + g) * N + c8);
            vc = *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const bf16 *>(p.C) + ((t0 + j) * p.G + g) * N + c8);
        }
        *reinterpret_cast<bf16x8 *>(Bs + j * SN + c8) = vb;
        *reinterpret_cast<bf16x8 *>(Cs + j * SN + c8) = vc;
    }
    __syncthreads();   // B and C rows in LDS

    // C B^T does not depend on the head: this wave's tiles (row band `band`,
    // column tiles JT half ..) are formed once.  W is only ever multiplied by
    // the head-independent B and C, so sum_h W_h is accumulated here and its
    // products with C and B are formed once, after the head loop.
    constexpr int JT = 4 / NH;   // 16-column tiles of the chunk per part
    f32x4 gt[JT], wacc[JT];
#pragma unroll
    for (int u = 0; u < JT; ++u) {
        const int jt = JT * half + u;
        gt[u] = wacc[u] = zero4();
#pragma unroll
        for (int k0 = 0; k0 < N; k0 += 32)
            gt[u] = mfma_bf16(gt[u], frag_row<SN>(Cs, row0 + li, k0, lg), frag_row<SN>(Bs, jt * 16 + li, k0, lg));
    }

    // one head's inputs in registers (loaded a head ahead; R issued later than
    // the rest, so that the loads do not all queue behind one barrier; the
    // states, read once, non-temporal)
    bf16x8 xr[XV], dyr[XV];
    f32x4 hr[SV], rr[SV];
    float dtr = 0.f;
    auto load_r = [&](int h) {
        const float *Rc = p.radj + ((long long)(o + c) * H + h) * PN;
#pragma unroll
        for (int k = 0; k < SV; ++k) {
            const int i = (tid + NTH * k) * 4;
            rr[k] = zero4();
            if (i < 4 * SP4) rr[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(Rc + i));
        }
    };
    auto load_head = [&](int h, bool with_r) {
#pragma unroll
        for (int k = 0; k < XV; ++k) {
            const int i = tid + NTH * k, j = i / (P / 8), c8 = (i % (P / 8)) * 8;
            xr[k] = dyr[k] = zero_frag<bf16x8>();
            if (i < XP && j < q) {
                xr[k] = *reinterpret_cast<const bf16x8 *>(xg + ((t0 + j) * H + h) * P + c8);
                dyr[k] = *reinterpret_cast<const bf16x8 *>(dyg + ((t0 + j) * H + h) * P + c8);
            }
        }
        const float *Hc = p.states + ((long long)(o + s + c) * H + h) * PN;
#pragma unroll
        for (int k = 0; k < SV; ++k) {
            const int i = (tid + NTH * k) * 4;
            hr[k] = zero4();
            if (i < 4 * SP4) hr[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(Hc + i));
        }
        if (wave == 0) dtr = lane < q ? p.dt[(t0 + lane) * (H / p.hsub) + h / p.hsub] : 0.f;
        if (with_r) load_r(h);
    };

    f32x4 dBacc[NT2], dCacc[NT2];
#pragma unroll
    for (int k = 0; k < NT2; ++k) dBacc[k] = dCacc[k] = zero4();

    if (hpg > 0) load_head(g * hpg, true);
    float ddt_sub = 0.f;   // ddt of a model head summed over its kernel heads (wave 0)
    for (int hh = 0; hh < hpg; ++hh) {
        const int h = g * hpg + hh;
        // Lane indices re-derived per head: the tiles span more LDS than a ds
        // offset reaches, and without this the compiler keeps every address
        // derived from them live across the loop and spills.
        int tid_ = threadIdx.x;
        asm volatile("" : "+v"(tid_));
        const int tid = tid_, lane = tid & 63, li = lane & 15, lg = lane >> 4;
        __syncthreads();   // the previous head's tiles are no longer read
        if (hh > 0) flush_dx(h - 1);
        // this head's registers into LDS; dy . x over the chunk from the same registers
        float dd = 0.f;
#pragma unroll
        for (int k = 0; k < XV; ++k) {
            const int i = tid + NTH * k, j = i / (P / 8), c8 = (i % (P / 8)) * 8;
            if (i < XP) {
                *reinterpret_cast<bf16x8 *>(xs + j * SP + c8) = xr[k];
                *reinterpret_cast<bf16x8 *>(dys + j * SP + c8) = dyr[k];
#pragma unroll
                for (int e = 0; e < 8; ++e) dd += (float)xr[k][e] * (float)dyr[k][e];
            }
        }
        float hrd = 0.f;   // <R_c, H_c>
#pragma unroll
        for (int k = 0; k < SV; ++k) {
            if (tid + NTH * k >= SP4) break;
            int pp, nn;
            state_piece_pos<P>(tid + NTH * k, pp, nn);
            bf16x4 a, b, cc, d;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                hrd += hr[k][e] * rr[k][e];
                a[e] = (bf16)hr[k][e];
                b[e] = (bf16)(hr[k][e] - (float)a[e]);
                cc[e] = (bf16)rr[k][e];
                d[e] = (bf16)(rr[k][e] - (float)cc[e]);
            }
            *reinterpret_cast<bf16x4 *>(Hh + pp * SN + nn) = a;
            *reinterpret_cast<bf16x4 *>(Hl + pp * SN + nn) = b;
            *reinterpret_cast<bf16x4 *>(Rh + pp * SN + nn) = cc;
            *reinterpret_cast<bf16x4 *>(Rl + pp * SN + nn) = d;
        }
        hrd = bwd_wave_sum(hrd);
        if (lane == 0) hrp[wave] = hrd;
        const float Ah = p.A[h / p.hsub];
        if (wave == 0) {
            const float sc = wave_inclusive_sum(dtr * Ah) * kLog2e;
            const float slast = __shfl(sc, 63, 64);
            s2[lane] = sc;
            dtv[lane] = dtr;
            ew[lane] = __builtin_amdgcn_exp2f(slast - sc);
            es[lane] = __builtin_amdgcn_exp2f(sc);
        }
        __syncthreads();
        if (hh + 1 < hpg) load_head(h + 1, false);   // in flight during this head's MFMAs

        // dY X^T for rows row0..row0+15, this part's columns; M, the W sum and the Z sums
        {
            f32x4 et[JT];
#pragma unroll
            for (int u = 0; u < JT; ++u) {
                const int jt = JT * half + u;
                et[u] = zero4();
#pragma unroll
                for (int k0 = 0; k0 < P; k0 += 32)
                    et[u] = mfma_bf16(et[u], frag_row<SP>(dys, row0 + li, k0, lg), frag_row<SP>(xs, jt * 16 + li, k0, lg));
            }
            float rz[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < JT; ++u) {
                const int j = (JT * half + u) * 16 + li;
                const float sj = s2[j], dj = dtv[j];
                float cz = 0.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = row0 + 4 * lg + r;
                    const float dec = j <= i ? __builtin_amdgcn_exp2f(s2[i] - sj) : 0.f;
                    const float z = gt[u][r] * et[u][r] * dec;
                    rz[r] += z * dj;
                    cz += z;
                    Ms[i * SQ + j] = (bf16)(gt[u][r] * dec * dj);
                    wacc[u][r] += et[u][r] * dec * dj;
                }
                cz += __shfl_xor(cz, 16, 64);
                cz += __shfl_xor(cz, 32, 64);
                if (lg == 0) colP[band][j] = cz;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                rz[r] = row_sum16(rz[r]);
                if (li == 0) rowP[half][row0 + 4 * lg + r] = rz[r];
            }
        }
        dd = bwd_wave_sum(dd);
        if (lane == 0) red[wave] = dd;
        __syncthreads();   // M, partial sums
        if (tid == 0) {
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) t += red[w];
            p.partD[(long long)ci * H + h] = t;
        }

        if (hh + 1 < hpg) load_r(h + 1);
        // dx = M^T dY + diag(w) B R^T + D dY (this band, this half's columns)
        const float Dh = p.D ? p.D[h / p.hsub] : 0.f;
        // computed transposed (rows head-dim, columns tokens), so that each lane
        // holds 4 consecutive head-dim entries of one token: one 8-byte dy read
        // and one 8-byte piece of the LDS dx rows per tile
#pragma unroll
        for (int u = 0; u < PT2; ++u) {
            const int pt = half * PT2 + u;
            f32x4 a1 = zero4(), a2 = zero4();
#pragma unroll
            for (int k0 = 0; k0 < Q; k0 += 32)
                a1 = mfma_bf16(a1, frag_col<SP>(dys, k0, pt * 16, li, lg), frag_col<SQ>(Ms, k0, row0, li, lg));
#pragma unroll
            for (int k0 = 0; k0 < N; k0 += 32)
                a2 = mfma_bf16(a2, frag_row<SN>(Rh, pt * 16 + li, k0, lg), frag_row<SN>(Bs, row0 + li, k0, lg));
            const int j = row0 + li, p0 = pt * 16 + 4 * lg;
            if (j < q) {
                const float wj = ew[j] * dtv[j];
                const bf16x4 dyv = *reinterpret_cast<const bf16x4 *>(dys + j * SP + p0);
                bf16x4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = (bf16)(a1[r] + wj * a2[r] + Dh * (float)dyv[r]);
                *reinterpret_cast<bf16x4 *>(dxs + j * SP + p0) = o;
            }
        }

        // dB, dC of this head (this half's columns) and the row dot products
        float ob[4] = {0.f, 0.f, 0.f, 0.f}, oc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NT2; ++u) {
            const int nt = half * NT2 + u;
            f32x4 xb = zero4(), yc = zero4();
#pragma unroll
            for (int k0 = 0; k0 < P; k0 += 32) {
                const bf16x8 xrow = frag_row<SP>(xs, row0 + li, k0, lg);
                xb = mfma_bf16(xb, xrow, frag_col<SN>(Rh, k0, nt * 16, li, lg));
                xb = mfma_bf16(xb, xrow, frag_col<SN>(Rl, k0, nt * 16, li, lg));
                const bf16x8 yrow = frag_row<SP>(dys, row0 + li, k0, lg);
                yc = mfma_bf16(yc, yrow, frag_col<SN>(Hh, k0, nt * 16, li, lg));
                yc = mfma_bf16(yc, yrow, frag_col<SN>(Hl, k0, nt * 16, li, lg));
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rw = row0 + 4 * lg + r, nn = nt * 16 + li;
                const float xbr = xb[r] * ew[rw], ycr = yc[r] * es[rw];
                dBacc[u][r] += dtv[rw] * xbr;
                dCacc[u][r] += ycr;
                ob[r] += xbr * (float)Bs[rw * SN + nn];
                oc[r] += ycr * (float)Cs[rw * SN + nn];
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            ob[r] = row_sum16(ob[r]);
            oc[r] = row_sum16(oc[r]);
            if (li == 0) {
                offBP[half][row0 + 4 * lg + r] = ob[r];
                offCP[half][row0 + 4 * lg + r] = oc[r];
            }
        }
        __syncthreads();

        if (wave == 0) {
            const int j = lane;
            const float d = dtv[j];
            const float cz = colP[0][j] + colP[1][j] + colP[2][j] + colP[3][j];
            float ob_ = 0.f, rz = 0.f, oc_ = 0.f;
#pragma unroll
            for (int u = 0; u < NH; ++u) {
                ob_ += offBP[u][j];
                rz += rowP[u][j];
                oc_ += offCP[u][j];
            }
            float hrs = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) hrs += hrp[w];
            // <R_c, H_{c+1}> = exp(s_last) <R_c, H_c> + <R_c, S_c>, and <R_c, S_c> = sum_j dt_j offB_j
            const float rh = __builtin_amdgcn_exp2f(s2[Q - 1]) * hrs + bwd_wave_sum(d * ob_);
            const float ds = rz - d * cz + oc_ - d * ob_ + (j == q - 1 ? rh : 0.f);
            const float tot = bwd_wave_sum(ds);
            const float da = tot - wave_inclusive_sum(ds) + ds;
            const float v = Ah * da + cz + ob_;
            ddt_sub = (h % p.hsub == 0) ? v : ddt_sub + v;   // the model head's sub-heads, in order
            if (j < q && h % p.hsub == p.hsub - 1) p.ddt[(t0 + j) * (H / p.hsub) + h / p.hsub] = ddt_sub;
            const float pa = bwd_wave_sum(d * da);
            if (lane == 0) p.partA[(long long)ci * H + h] = pa;
        }
    }

    // diagonal parts of dB and dC: (sum_h W_h)^T C and (sum_h W_h) B, with the
    // sum as a split bf16 pair (high parts in Ms, remainders in Ws)
    __syncthreads();   // every wave is done with the last head's tiles
    if (hpg > 0) flush_dx(g * hpg + hpg - 1);
#pragma unroll
    for (int u = 0; u < JT; ++u) {
        const int j = (JT * half + u) * 16 + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = row0 + 4 * lg + r;
            const bf16 hi = (bf16)wacc[u][r];
            Ms[i * SQ + j] = hi;
            Ws[i * SQ + j] = (bf16)(wacc[u][r] - (float)hi);
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NT2; ++u) {
        const int nt = half * NT2 + u;
        f32x4 db = zero4(), dc = zero4();
#pragma unroll
        for (int k0 = 0; k0 < Q; k0 += 32) {
            const bf16x8 cf = frag_col<SN>(Cs, k0, nt * 16, li, lg), bfr = frag_col<SN>(Bs, k0, nt * 16, li, lg);
            db = mfma_bf16(db, frag_col<SQ>(Ms, k0, row0, li, lg), cf);
            db = mfma_bf16(db, frag_col<SQ>(Ws, k0, row0, li, lg), cf);
            dc = mfma_bf16(dc, frag_row<SQ>(Ms, row0 + li, k0, lg), bfr);
            dc = mfma_bf16(dc, frag_row<SQ>(Ws, row0 + li, k0, lg), bfr);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            dBacc[u][r] += db[r];
            dCacc[u][r] += dc[r];
        }
    }
#pragma unroll
    for (int u = 0; u < NT2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rw = row0 + 4 * lg + r, nn = (half * NT2 + u) * 16 + li;
            if (rw < q) {
                p.dB[((t0 + rw) * p.G + g) * N + nn] = dBacc[u][r];
                p.dC[((t0 + rw) * p.G + g) * N + nn] = dCacc[u][r];
            }
        }
}

// bf16 version of the chunk-sequential scans for headdim and dstate >= 32.
// The two scans are independent, so one launch runs both (twice the
// workgroups of either: the chains are latency-bound), and its register
// budget allows three workgroups per compute unit.  The next chunk's rows
// and dt are loaded into registers while the current chunk is computed; u is
// scaled by the decay weights once per chunk and kept in LDS as a split bf16
// pair, and both MFMA operands are read in the K-slot order with transposing
// LDS reads.  Every global access goes through a buffer resource, rows past
// the chunk (and a missing state) given as out-of-range offsets that read
// zero, so that each path issues the same memory operations: the compiler
// then waits for the prefetched rows alone, and the state stores, issued
// after them, stay in flight while the next chunk is staged.
template <int P, int N, int MODE>
__device__ __forceinline__ void scan_bf16_chain(const BwdParams &p, int unit, bf16 *sv, bf16 *uh, bf16 *ul,
                                                float *swt, float *salpha) {
    constexpr int Q = kBwdQ;
    constexpr int PT = P / 16, NT = N / 16, TILES = PT * NT;
    constexpr int TPW = (TILES + 3) / 4;
    constexpr int SP = P + 8, SN = N + 8;
    constexpr int UV = Q * P / 8 / 256;     // 16-byte pieces of u per thread (P >= 32: 1 or 2)
    constexpr int VV = Q * N / 8 / 256;     // likewise for v (1, 2 or 4)
    static_assert(UV >= 1 && VV >= 1, "shape too small for this kernel");
    constexpr int PN = P * N;
    // (wave masked to its 0..3 range: the tile tests below then fold away)
    const int tid = threadIdx.x, lane = tid & 63, wave = (tid >> 6) & 3;
    const int li = lane & 15, lg = lane >> 4;
    const int s = unit / p.H, h = unit - s * p.H;
    const int g = h / (p.H / p.G);
    const int o = p.seq_chunk_start[s];
    const int nc = p.seq_chunk_start[s + 1] - o;
    const bf16 *ug = reinterpret_cast<const bf16 *>(MODE == 0 ? p.x : p.dy);
    const bf16 *vg = reinterpret_cast<const bf16 *>(MODE == 0 ? p.B : p.C);
    const float Ah = p.A[h / p.hsub];
    const int HP = p.H * P, GN = p.G * N, HD = p.H / p.hsub;   // row strides of u, v and dt

    // Wave w holds state tiles t = w + 4 k, (pt, nt) = (t % PT, t / PT):
    // element r of tile k is state[pt*16 + li][nt*16 + 4 lg + r].
    auto tile_off = [&](int k) {   // byte offset of this lane's 4 floats of tile k, row-major state
        const int t = wave + 4 * k;
        return ((t % PT) * 16 + li) * N * 4 + ((t / PT) * 16 + 4 * lg) * 4;
    };

    // the sequence's chunks are consecutive Q-token pieces from its first token
    long long seq_t0 = 0;
    int seq_len = 0;
    if (nc > 0) {
        const int4 f = p.chunks[o], l = p.chunks[o + nc - 1];
        seq_t0 = f.y;
        seq_len = l.y + l.z - f.y;
    }
    // registers of one chunk: u and v pieces (row j, 8 columns) and dt; a
    // chunk index outside the sequence loads zeros
    bf16x8 ur[UV], vr[VV];
    float dtr;
    auto load_chunk = [&](int c) {
        const bool in = c >= 0 && c < nc;
        const int q = in ? min(Q, seq_len - c * Q) : 0;
        const long long t0 = seq_t0 + (long long)(in ? c : 0) * Q;
        // (u non-temporal: the head's rows are read once here, and the L2
        // keeps the chunk's B or C rows that the group's other heads read too)
        const __amdgpu_buffer_rsrc_t ru = buf_rsrc(ug + t0 * HP, q * HP * 2);
        const __amdgpu_buffer_rsrc_t rv = buf_rsrc(vg + t0 * GN, q * GN * 2);
        const __amdgpu_buffer_rsrc_t rd = buf_rsrc(p.dt + t0 * HD, q * HD * 4);
        // issued in the order of first use (dt, v, u), the same on every
        // path into the chunk loop, so that the waits at its top are exact
        dtr = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, (lane * HD + h / p.hsub) * 4, 0, 0));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < VV; ++k) {
            const int i = tid + 256 * k, j = i / (N / 8), c8 = (i % (N / 8)) * 8;
            vr[k] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, (j * GN + g * N + c8) * 2, 0, 0));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < UV; ++k) {
            const int i = tid + 256 * k, j = i / (P / 8), c8 = (i % (P / 8)) * 8;
            ur[k] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ru, (j * HP + h * P + c8) * 2, 0, kStream));
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    load_chunk(MODE == 0 ? 0 : nc - 1);

    f32x4 st[TPW];
    {
        const float *st0 = MODE == 0 ? p.init_state : p.dfinal;
        const __amdgpu_buffer_rsrc_t r0 =
            buf_rsrc(st0 ? st0 + ((long long)s * p.H + h) * PN : nullptr, st0 ? PN * 4 : 0);
#pragma unroll
        for (int k = 0; k < TPW; ++k)
            st[k] = wave + 4 * k < TILES
                ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r0, tile_off(k), 0, 0))
                : zero4();
    }
    // the workspace's states in the tile order of state_piece_pos (tile t, this
    // lane's piece), non-temporal: only the chunk kernel reads them, after this
    // launch, and the L2 keeps the B or C rows a group's heads share instead;
    // the initial-state gradient row-major (null: no store)
    auto store_state = [&](float *dst, bool row_major = false) {
        const __amdgpu_buffer_rsrc_t r = buf_rsrc(dst, dst ? PN * 4 : 0);
#pragma unroll
        for (int k = 0; k < TPW; ++k)
            if (wave + 4 * k < TILES)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, st[k]), r,
                                                       row_major ? tile_off(k) : ((wave + 4 * k) * 64 + lane) * 16, 0, kStream);
    };
    if (MODE == 0) store_state(p.states + ((long long)(o + s) * p.H + h) * PN);

    for (int step = 0; step < nc; ++step) {
        const int c = MODE == 0 ? step : nc - 1 - step;
        // v rows and the weights of this chunk into LDS
#pragma unroll
        for (int k = 0; k < VV; ++k) {
            const int i = tid + 256 * k, j = i / (N / 8), c8 = (i % (N / 8)) * 8;
            *reinterpret_cast<bf16x8 *>(sv + j * SN + c8) = vr[k];
        }
        if (wave == 0) {
            const float sc = wave_inclusive_sum(dtr * Ah) * kLog2e;   // s * log2(e)
            const float slast = __shfl(sc, 63, 64);
            swt[lane] = MODE == 0 ? __builtin_amdgcn_exp2f(slast - sc) * dtr : __builtin_amdgcn_exp2f(sc);
            if (lane == 0) *salpha = __builtin_amdgcn_exp2f(slast);
        }
        __syncthreads();
        // u scaled by the weights, as a split pair
#pragma unroll
        for (int k = 0; k < UV; ++k) {
            const int i = tid + 256 * k, j = i / (P / 8), c8 = (i % (P / 8)) * 8;
            const float w = swt[j];
            bf16x8 hi, lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = (float)ur[k][e] * w;
                hi[e] = (bf16)v;
                lo[e] = (bf16)(v - (float)hi[e]);
            }
            *reinterpret_cast<bf16x8 *>(uh + j * SP + c8) = hi;
            *reinterpret_cast<bf16x8 *>(ul + j * SP + c8) = lo;
        }
        const float alpha = *salpha;
        __syncthreads();
        load_chunk(MODE == 0 ? c + 1 : c - 1);   // in flight during the MFMAs (zeros past the end)
        if (MODE == 1) store_state(p.radj + ((long long)(o + c) * p.H + h) * PN);
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int t = wave + 4 * k;
            if (t < TILES) {
                const int pt = t % PT, nt = t / PT;
                // rows n (A operand v^T), columns p (B operand: u scaled by the weights)
                f32x4 acc = zero4();
#pragma unroll
                for (int k0 = 0; k0 < Q; k0 += 32) {
                    const bf16x8 a = frag_col<SN>(sv, k0, nt * 16, li, lg);
                    acc = mfma_bf16(acc, a, frag_col<SP>(uh, k0, pt * 16, li, lg));
                    acc = mfma_bf16(acc, a, frag_col<SP>(ul, k0, pt * 16, li, lg));
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) st[k][r] = alpha * st[k][r] + acc[r];
            }
        }
        if (MODE == 0) store_state(p.states + ((long long)(o + s + c + 1) * p.H + h) * PN);
        __syncthreads();   // the LDS tiles are rewritten by the next chunk
    }
    if (MODE == 1) store_state(p.dinit ? p.dinit + ((long long)s * p.H + h) * PN : nullptr, true);
}

// Blocks [0, nseq H) run the forward boundary states (MODE 0), blocks
// [nseq H, 2 nseq H) the reverse chain (MODE 1).
template <int P, int N>
__global__ __launch_bounds__(256, 3) void ssd_bwd_scan_bf16_kernel(BwdParams p) {
    constexpr int Q = kBwdQ;
    __shared__ __attribute__((aligned(16))) bf16 sv[Q * (N + 8)];
    __shared__ __attribute__((aligned(16))) bf16 uh[Q * (P + 8)];
    __shared__ __attribute__((aligned(16))) bf16 ul[Q * (P + 8)];
    __shared__ float swt[Q];
    __shared__ float salpha;
    const int units = p.nseq * p.H;
    if ((int)blockIdx.x < units)
        scan_bf16_chain<P, N, 0>(p, blockIdx.x, sv, uh, ul, swt, &salpha);
    else
        scan_bf16_chain<P, N, 1>(p, (int)blockIdx.x - units, sv, uh, ul, swt, &salpha);
}

// dA[h], dD[h]: sums of the per-chunk partials of the model head's kernel
// heads, one workgroup per model head, in a fixed order (strided partial
// sums, then a fixed tree).
__global__ __launch_bounds__(256) void ssd_bwd_reduce_kernel(BwdParams p) {
    __shared__ float red[2][4];
    const int h = blockIdx.x;
    const int n_chunks = p.seq_chunk_start[p.nseq];
    float a = 0.f, d = 0.f;
    for (int c = threadIdx.x; c < n_chunks; c += 256) {
        for (int u = 0; u < p.hsub; ++u) {
            a += p.partA[(long long)c * p.H + h * p.hsub + u];
            d += p.partD[(long long)c * p.H + h * p.hsub + u];
        }
    }
    a = bwd_wave_sum(a);
    d = bwd_wave_sum(d);
    if ((threadIdx.x & 63) == 0) {
        red[0][threadIdx.x >> 6] = a;
        red[1][threadIdx.x >> 6] = d;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        p.dA[h] = red[0][0] + red[0][1] + red[0][2] + red[0][3];
        p.dD[h] = red[1][0] + red[1][1] + red[1][2] + red[1][3];
    }
}

}  // namespace ssd

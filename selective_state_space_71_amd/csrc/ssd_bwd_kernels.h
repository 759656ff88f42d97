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
// Kernels: ssd_bwd_prep_kernel (chunk table), ssd_bwd_scan_kernel (forward
// boundary states H_c, or the reverse chain R_c; one workgroup per
// (sequence, head), chunk-sequential), ssd_bwd_chunk_kernel (everything
// else; one workgroup per (chunk, group), looping over the group's heads so
// that dB and dC accumulate in registers without atomics) and
// ssd_bwd_reduce_kernel (dA and dD from per-chunk partials, in a fixed order).
#pragma once

#include "ssd_device.h"

namespace ssd {

constexpr int kBwdQ = 64;         // tokens per chunk of the backward pass
constexpr float kBwdLog2e = 1.4426950408889634f;

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
    float *states;                // [n_chunks + nseq][H][P][N]: H_0 .. H_T of every sequence
    float *radj;                  // [n_chunks][H][P][N]: R_c
    float *partA, *partD;         // [n_chunks][H]
    int H, G, nseq;
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

__device__ __forceinline__ float bwd_wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Inclusive prefix sum over the 64 lanes of a wave (log-step shuffles).
__device__ __forceinline__ float bwd_wave_scan(float v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float t = __shfl_up(v, off, 64);
        if (lane >= off) v += t;
    }
    return v;
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
    const float Ah = p.A[h];

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
            const float d = lane < q ? p.dt[(t0 + lane) * p.H + h] : 0.f;
            const float sc = bwd_wave_scan(d * Ah, lane) * kBwdLog2e;   // s * log2(e)
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

    for (int hh = 0; hh < hpg; ++hh) {
        const int h = g * hpg + hh;
        __syncthreads();   // the previous head's tiles are no longer read
        stage_rows<IO, P>(xs, reinterpret_cast<const IO *>(p.x), t0, q, (long long)H * P, (long long)h * P, tid);
        stage_rows<IO, P>(dys, reinterpret_cast<const IO *>(p.dy), t0, q, (long long)H * P, (long long)h * P, tid);
        const float *Hc = p.states + ((long long)(o + s + c) * H + h) * PN;
        const float *Hn = p.states + ((long long)(o + s + c + 1) * H + h) * PN;
        const float *Rc = p.radj + ((long long)(o + c) * H + h) * PN;
        float rh = 0.f;
        for (int i = tid; i < P * N; i += 256) {
            const float r = Rc[i];
            Hs[i] = Hc[i];
            Rs[i] = r;
            rh += r * Hn[i];
        }
        const float Ah = p.A[h];
        if (wave == 0) {
            const float d = lane < q ? p.dt[(t0 + lane) * H + h] : 0.f;
            const float sc = bwd_wave_scan(d * Ah, lane) * kBwdLog2e;
            const float slast = __shfl(sc, 63, 64);
            s2[lane] = sc;
            dtv[lane] = d;
            ew[lane] = __builtin_amdgcn_exp2f(slast - sc);
            es[lane] = __builtin_amdgcn_exp2f(sc);
        }
        rh = block_sum(rh, red);   // (its barriers also publish the tiles above)

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
        const float Dh = p.D ? p.D[h] : 0.f;
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
            float ds = rowZ[j] - d * colZ[j] + offC[j] - d * offB[j] + (j == q - 1 ? rh : 0.f);
            const float tot = bwd_wave_sum(ds);
            const float da = tot - bwd_wave_scan(ds, lane) + ds;    // sum over i >= j
            if (j < q) p.ddt[(t0 + j) * H + h] = Ah * da + colZ[j] + offB[j];
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

// dA[h], dD[h]: sums of the per-chunk partials in chunk order.
__global__ __launch_bounds__(256) void ssd_bwd_reduce_kernel(BwdParams p) {
    const int h = blockIdx.x * 256 + threadIdx.x;
    if (h >= p.H) return;
    const int n_chunks = p.seq_chunk_start[p.nseq];
    float a = 0.f, d = 0.f;
    for (int c = 0; c < n_chunks; ++c) {
        a += p.partA[(long long)c * p.H + h];
        d += p.partD[(long long)c * p.H + h];
    }
    p.dA[h] = a;
    p.dD[h] = d;
}

}  // namespace ssd

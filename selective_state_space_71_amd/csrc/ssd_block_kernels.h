// ssd_block_kernels.h -- the block prologue and epilogue around the SSD layer
// (gfx950 / CDNA4), both streaming kernels bound by HBM bandwidth.
//
// The Mamba block (feghi.github.io Mamba review, section 5, the block figure
// read bottom to top) sends one projected branch through a short causal
// convolution and an activation into the selective SSM and turns the other
// branch into a multiplicative gate on its output; the Mamba-2 review
// (dimensionstp.github.io "Transformers are SSMs Review", section 3-2, item 5)
// adds a NormFormer-style extra normalization there.
//
//   ssd_conv1d_kernel   depthwise causal convolution (width 1..4 taps, the
//                       last tap on the current token) of the fused x | B | C
//                       projection, optional bias and SiLU, written straight
//                       into the x, B and C layouts the SSD forward reads.
//   ssd_gated_norm_kernel  RMSNorm over channel groups of y * silu(z) (or of y,
//                       gated after the norm), times a per-channel weight.
#pragma once

#include "ssd_device.h"

namespace ssd {

constexpr float kLog2eF = 1.4426950408889634f;

// SiLU v * logistic(v) = v / (1 + exp(-v)); exp(-v) overflows to +inf for
// v << 0, which gives -0 (the limit).
__device__ __forceinline__ float silu_f(float v) {
    return v * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-v * kLog2eF));
}

// 8 consecutive channels of one token: 16 bytes (bf16) or 32 bytes (fp32).
template <typename IO> struct Chan8;
template <> struct Chan8<bf16> {
    typedef bf16x8 T;
};
template <> struct Chan8<float> {
    typedef f32x8 T;
};

template <typename IO>
__device__ __forceinline__ void load8(const IO *p, float (&v)[8]) {
    const typename Chan8<IO>::T t = *reinterpret_cast<const typename Chan8<IO>::T *>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = to_f32(t[e]);
}

template <typename IO>
__device__ __forceinline__ void store8(IO *p, const float (&v)[8]) {
    typename Chan8<IO>::T t;
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = from_f32<IO>(v[e]);
    *reinterpret_cast<typename Chan8<IO>::T *>(p) = t;
}

// The same as a streaming (non-temporal) store: data written once and not
// read again by this kernel.
template <typename IO>
__device__ __forceinline__ void store8_stream(IO *p, const float (&v)[8]) {
    typename Chan8<IO>::T t;
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = from_f32<IO>(v[e]);
    __builtin_nontemporal_store(t, reinterpret_cast<typename Chan8<IO>::T *>(p));
}

// ---------------------------------------------------------------------------
// Causal depthwise convolution.
struct ConvParams {
    const void *xbc;        // [tokens, Cc] io, channels x | B | C
    const float *w;         // [Cc, W] fp32
    const float *bias;      // [Cc] fp32 or null
    const void *state_in;   // [nseq, W-1, Cc] io or null (zeros)
    const int *cu_seqlens;  // [nseq + 1] or null (dense: each batch row a sequence)
    void *x;                // [tokens, HP] io
    void *B;                // [tokens, GN] io
    void *C;                // [tokens, GN] io
    void *state_out;        // [nseq, W-1, Cc] io or null
    long long tokens;
    int seqlen, nseq, Cc, HP, GN;
    int silu;
    int run;                // tokens per thread
};

// Thread (chunk, run): channels 8*chunk .. 8*chunk+7 of tokens
// [run*T, run*T + T).  A wave covers 64 consecutive chunks, so every token
// row is read and written as contiguous 1 KB (bf16) pieces.  Rows stream in
// batches of 16 tokens (all 16 loads in flight before the first is used),
// with non-temporal loads and stores: the input is read once (the W-1 rows
// before a run are ordinary loads) and the outputs are not read here.  The run is cut
// at sequence boundaries; at a sequence's start the width-1 previous inputs
// come from the sequence's initial state (or are zero), and the thread that
// holds a sequence's last token writes its final state.
template <typename IO, int W>
__global__ __launch_bounds__(256) void ssd_conv1d_kernel(ConvParams p) {
    const int chunk = blockIdx.x * 64 + (threadIdx.x & 63);
    const long long run = (long long)blockIdx.y * 4 + (threadIdx.x >> 6);
    const int n_chunks = p.Cc / 8;
    if (chunk >= n_chunks) return;
    const int c0 = chunk * 8;
    const IO *in = reinterpret_cast<const IO *>(p.xbc);
    const IO *st_in = reinterpret_cast<const IO *>(p.state_in);
    IO *st_out = reinterpret_cast<IO *>(p.state_out);

    // output tensor and column of this chunk (a chunk never straddles x | B | C)
    IO *dst;
    int dst_stride, dst_col;
    if (c0 < p.HP) {
        dst = reinterpret_cast<IO *>(p.x), dst_stride = p.HP, dst_col = c0;
    } else if (c0 < p.HP + p.GN) {
        dst = reinterpret_cast<IO *>(p.B), dst_stride = p.GN, dst_col = c0 - p.HP;
    } else {
        dst = reinterpret_cast<IO *>(p.C), dst_stride = p.GN, dst_col = c0 - p.HP - p.GN;
    }

    // Empty packed sequences: the final state is the initial one (or zero).
    if (p.cu_seqlens && p.state_out && blockIdx.y == 0 && (threadIdx.x >> 6) == 0) {
        for (int s = 0; s < p.nseq; ++s) {
            if (p.cu_seqlens[s + 1] != p.cu_seqlens[s]) continue;
            for (int j = 0; j < W - 1; ++j) {
                float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                if (st_in) load8(st_in + ((long long)s * (W - 1) + j) * p.Cc + c0, v);
                store8(st_out + ((long long)s * (W - 1) + j) * p.Cc + c0, v);
            }
        }
    }

    const long long t_begin = run * p.run;
    if (t_begin >= p.tokens) return;
    const long long t_end = min(t_begin + p.run, p.tokens);

    float wt[W][8], bs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
        for (int k = 0; k < W; ++k) wt[k][e] = p.w[(c0 + e) * W + k];
        bs[e] = p.bias ? p.bias[c0 + e] : 0.f;
    }

    long long t = t_begin;
    while (t < t_end) {
        // the sequence holding token t: index s, tokens [a, e)
        int s;
        long long a, e;
        if (p.cu_seqlens) {
            int lo = 0, hi = p.nseq - 1;   // first s with cu[s + 1] > t
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (p.cu_seqlens[mid + 1] > t) hi = mid; else lo = mid + 1;
            }
            s = lo;
            a = p.cu_seqlens[s];
            e = p.cu_seqlens[s + 1];
        } else {
            s = (int)(t / p.seqlen);
            a = (long long)s * p.seqlen;
            e = a + p.seqlen;
        }
        const long long seg_end = min(e, t_end);
        // window: win[j] is the input of token t - (W - 1) + j
        float win[W > 1 ? W - 1 : 1][8];
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            const long long tau = t - (W - 1) + j;
#pragma unroll
            for (int q = 0; q < 8; ++q) win[j][q] = 0.f;
            if (tau >= a) {
                load8(in + tau * p.Cc + c0, win[j]);
            } else if (st_in) {
                const long long r = (W - 1) - (a - tau);   // row of the initial state
                load8(st_in + ((long long)s * (W - 1) + r) * p.Cc + c0, win[j]);
            }
        }
        // tokens in batches of TB: all TB rows are loaded before any is used
        constexpr int TB = 16;
        auto step = [&](const float (&cur)[8], long long tt) {
            float o[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                float acc = bs[q];
#pragma unroll
                for (int k = 0; k < W - 1; ++k) acc += wt[k][q] * win[k][q];
                acc += wt[W - 1][q] * cur[q];
                o[q] = p.silu ? silu_f(acc) : acc;
            }
            store8_stream(dst + tt * dst_stride + dst_col, o);
#pragma unroll
            for (int k = 0; k + 1 < W - 1; ++k)
#pragma unroll
                for (int q = 0; q < 8; ++q) win[k][q] = win[k + 1][q];
            if constexpr (W > 1) {
#pragma unroll
                for (int q = 0; q < 8; ++q) win[W - 2][q] = cur[q];
            }
        };
        for (; t + TB <= seg_end; t += TB) {
            typename Chan8<IO>::T raw[TB];
#pragma unroll
            for (int j = 0; j < TB; ++j)
                raw[j] = __builtin_nontemporal_load(reinterpret_cast<const typename Chan8<IO>::T *>(in + (t + j) * p.Cc + c0));
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                float cur[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) cur[q] = to_f32(raw[j][q]);
                step(cur, t + j);
            }
        }
        for (; t < seg_end; ++t) {
            float cur[8];
            load8(in + t * p.Cc + c0, cur);
            step(cur, t);
        }
        if (seg_end == e && st_out) {
#pragma unroll
            for (int j = 0; j < W - 1; ++j) store8(st_out + ((long long)s * (W - 1) + j) * p.Cc + c0, win[j]);
        }
    }
}

// ---------------------------------------------------------------------------
// Gated RMSNorm.
struct NormParams {
    const void *y;      // [rows, dim] io
    const void *z;      // [rows, dim] io or null (no gate)
    const float *w;     // [dim] fp32
    void *out;          // [rows, dim] io (may be y or z itself)
    long long units;    // rows * groups
    int dim, gs, groups;
    float eps;
};

// Sum over the 64 lanes of a wave (a fixed butterfly order: deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// One wave per (row, group): lane l holds channels 512 c + 8 l .. + 7 of the
// group for c < NCH.  All loads (y, z and the weight) are issued before any
// is used; the group is reduced and then scaled and written, so `out` may be
// `y` or `z` itself.  MODE: 0 no gate, 1 norm of y * silu(z), 2 norm of y
// gated by silu(z) afterwards.
template <typename IO, int NCH, int MODE>
__global__ __launch_bounds__(256) void ssd_gated_norm_kernel(NormParams p) {
    const long long unit = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (unit >= p.units) return;
    const int lane = threadIdx.x & 63;
    const long long row = unit / p.groups;
    const int g = (int)(unit - row * p.groups);
    const long long base = row * p.dim + (long long)g * p.gs;
    const IO *yp = reinterpret_cast<const IO *>(p.y) + base;
    const IO *zp = reinterpret_cast<const IO *>(p.z) + base;
    const float *wp = p.w + (long long)g * p.gs;
    IO *op = reinterpret_cast<IO *>(p.out) + base;
    typedef typename Chan8<IO>::T V;
    V yv[NCH], zv[NCH];
    f32x4 wv[NCH][2];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int ch = 512 * c + 8 * lane;
        if (c + 1 < NCH || ch < p.gs) {   // only the last chunk can be partial
            yv[c] = *reinterpret_cast<const V *>(yp + ch);
            if constexpr (MODE != 0) zv[c] = *reinterpret_cast<const V *>(zp + ch);
            wv[c][0] = *reinterpret_cast<const f32x4 *>(wp + ch);
            wv[c][1] = *reinterpret_cast<const f32x4 *>(wp + ch + 4);
        }
    }
    float v[NCH][8];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int ch = 512 * c + 8 * lane;
        const bool live = c + 1 < NCH || ch < p.gs;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float t = live ? to_f32(yv[c][e]) : 0.f;
            if constexpr (MODE == 1) t *= live ? silu_f(to_f32(zv[c][e])) : 0.f;
            v[c][e] = t;
            ss += t * t;
        }
    }
    ss = wave_sum(ss);
    const float rinv = __builtin_amdgcn_rsqf(ss / (float)p.gs + p.eps);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int ch = 512 * c + 8 * lane;
        if (c + 1 < NCH || ch < p.gs) {
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                o[e] = v[c][e] * rinv * wv[c][e >> 2][e & 3];
                if constexpr (MODE == 2) o[e] *= silu_f(to_f32(zv[c][e]));
            }
            store8(op + ch, o);
        }
    }
}

}  // namespace ssd

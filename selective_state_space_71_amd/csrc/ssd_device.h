// ssd_device.h -- device helpers shared by the SSD kernels (gfx950 / CDNA4).
//
// MFMA fragments.  All contractions use the 16x16 output tile of the gfx950
// matrix cores with a K step of 32:
//   bf16 io: one v_mfma_f32_16x16x32_bf16 per K step;
//   fp32 io: eight v_mfma_f32_16x16x4_f32 per K step (one per fragment slot).
// A fragment is 8 values per lane.  Lane l has group g = l / 16 and index
// i = l % 16.  For the A operand (rows x K) lane l holds row i; for the B
// operand (K x cols) it holds column i.  Slot e (0..7) of group g carries
// the K index kmap(g, e); any kmap works as long as A and B use the same one,
// because the product sums over every (g, e) pair.  The accumulator holds
// D[4g + r][i] in element r (r = 0..3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

template <typename T> struct Io;

template <> struct Io<bf16> {
    typedef bf16x8 Frag;
    typedef bf16x4 Half;
    static __device__ __forceinline__ f32x4 mfma(f32x4 acc, Frag a, Frag b) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
};

template <> struct Io<float> {
    typedef f32x8 Frag;
    typedef f32x4 Half;
    static __device__ __forceinline__ f32x4 mfma(f32x4 acc, Frag a, Frag b) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
        return acc;
    }
};

__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }

// Buffer resource over `bytes` bytes at `base`: reads past the end return 0
// and writes past it are dropped (0 bytes: every access is a no-op).  The
// kernels' loops make their global accesses through these, with out-of-range
// offsets instead of branches, so that every path issues the same vector
// memory operations: the compiler then knows how many follow each load and
// waits for exactly the ones a use needs (operations issued under a branch
// make it wait for whatever might have been issued).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

// Cache-policy operand of a buffer access that streams data used once (a
// head's x or dy rows, the y rows): non-temporal, so that these lines are
// the first the XCD's L2 gives up and the data that is read again (states
// handed from chunk to chunk, the B and C rows a group's heads share) stays.
constexpr int kStream = 2;   // nt

template <typename Frag> __device__ __forceinline__ Frag zero_frag() {
    Frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = 0;
    return f;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Transposing LDS read of 16-bit data (gfx950 ds_read_b64_tr_b16): inside a
// 16-lane group, lane i receives column i%16 of the four rows addressed by
// lanes 4e..4e+3, where lane 4e+c points at columns [4c, 4c+4) of row e.
__device__ __forceinline__ bf16x4 lds_read_tr16(const bf16 *p) {
    i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)(p));
    return __builtin_bit_cast(bf16x4, v);
}

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2f_fast(float v) { return __builtin_amdgcn_exp2f(v); }

// v + (v of the lane the DPP control `ctrl` selects); lanes without a source
// (or outside `row_mask`) add 0.
template <int ctrl, int row_mask>
__device__ __forceinline__ float dpp_add(float v) {
    const int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, row_mask, 0xF, true);
    return v + __builtin_bit_cast(float, t);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: four
// shifts inside each 16-lane row, then the last lane of rows 0 and 2 into
// rows 1 and 3, then lane 31 into rows 2 and 3.
__device__ __forceinline__ float wave_inclusive_sum(float v) {
    v = dpp_add<0x111, 0xF>(v);   // row_shr:1
    v = dpp_add<0x112, 0xF>(v);   // row_shr:2
    v = dpp_add<0x114, 0xF>(v);   // row_shr:4
    v = dpp_add<0x118, 0xF>(v);   // row_shr:8
    v = dpp_add<0x142, 0xA>(v);   // row_bcast:15
    v = dpp_add<0x143, 0xC>(v);   // row_bcast:31
    return v;
}

// Sum over the 16 lanes of each row of the wave, in every lane of the row:
// pairs, quads, then the mirrored half and the mirrored row.
__device__ __forceinline__ float row_sum16(float v) {
    v = dpp_add<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
    v = dpp_add<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
    v = dpp_add<0x141, 0xF>(v);   // row_half_mirror
    v = dpp_add<0x140, 0xF>(v);   // row_mirror
    return v;
}

// Step-size preprocessing (see ssd_dt_opts_t): dt = clamp(softplus(dt + bias)).
struct DtProc {
    const float *bias;   // [nheads] or null
    bool on;             // any preprocessing at all
    bool softplus;
    float lo, hi;
    __device__ __forceinline__ float apply(float v, float b) const {
        v += b;
        if (softplus) v = v > 20.f ? v : log1pf(expf(v));
        return fminf(fmaxf(v, lo), hi);
    }
};

}  // namespace ssd

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
// (D_h x is formed inside Y_diag: D_h is added to the diagonal of the mask.)
//
// Decay by blocks.  The chunk is cut into blocks of 64 tokens; e_b is the
// cumulative sum at the last token of block b.  Each head's x is staged twice
// in LDS: as is, and as
//   xh_j = exp(e_b(j) - s_j) dt_j x_j            (a factor <= 1 per token).
// For a row i in block R and a column j in an earlier block b < R,
//   exp(s_i - s_j) = exp(s_i - e_{R-1}) * exp(e_{R-1} - e_b) * exp(e_b - s_j),
// every factor <= 1 (A <= 0, dt >= 0), so the part of Y_diag that lies left of
// the row's own block is
//   diag(exp(s_i - e_{R-1})) sum_{b<R} exp(e_{R-1} - e_b) G[i, block b] xh_b,
// a sum that is accumulated block by block (Horner's rule: scale the
// accumulator by the block decay exp(e_b - e_{b-1}), then add block b's
// product).  Those products take the C B^T tiles straight from registers as
// MFMA operands: no per-element work.  Only the row's own 64-token block is
// built explicitly (decay-weighted mask, with a per-element exponential on the
// diagonal 16 x 16 tiles and row x column factors on the others).  The chunk
// state uses the same staged xh with the same recurrence over all blocks:
//   S_c = sum_b exp(e_last - e_b) B_b^T xh_b.
//
// Work decomposition.  A workgroup (8 waves) owns one chunk of one B/C group
// and a slice of that group's heads.  C B^T depends only on the chunk and the
// group (heads of a group share B and C: the multi-input head pattern of
// section 3-2(5)), so it is formed once per workgroup and kept in registers:
// wave w owns the 16-row tiles w and 15 - w of the chunk (balanced causal
// work) and holds their lower-triangular C B^T tiles.  The B^T operands of the
// chunk state (the wave's state columns over the whole chunk) are also
// head-independent and stay in registers where they fit.  Per head only x and
// dt are loaded (prefetched during the previous head).
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
// Exponentials are evaluated as exp2 of log2(e)-scaled sums.  Accumulation and
// the boundary state are fp32.
#pragma once

#include <climits>
#include <type_traits>

#include "ssd_device.h"

// Debug build switch (0 in the library; 1 in the race-widening build).
#ifndef SSD_RACE_WIDEN
#define SSD_RACE_WIDEN 0
#endif

namespace ssd {

// Race-widening debug build: before storing its part of H_{c+1}, each
// producer wave sleeps a time that varies with the unit, the chunk and the
// wave (0 to 15 x 512 cycles).  The parts of one state then land far apart,
// so a consumer that read before the counter reached all kWaves increments,
// or whose loads could be served from a stale copy, would see old values.
// The arithmetic is unchanged: outputs must stay bitwise equal to the
// ordinary build's.
__device__ __forceinline__ void race_widen_delay(int unit, int cloc, int wave) {
    const int n = (unit * 7 + cloc * 13 + wave * 5) & 15;
    for (int k = 0; k < n; ++k) __builtin_amdgcn_s_sleep(8);
}

// Mark in a chunk entry's length field: the sequence's last chunk, whose
// boundary state is the final state.
constexpr int kLastChunk = 1 << 30;

// Order of a boundary state in the state buffer.  Handed from chunk to
// chunk it follows the accumulator's lane order, tile after tile: tile
// (nt, pt) is 64 pieces of 4 floats, piece l holding state[16 pt + l % 16]
// [16 nt + 4 (l / 16) + 0..3], so a wave's load or store of a tile is 1 KB of
// consecutive bytes.  The initial and the final state are row-major.
template <int P>
__device__ __forceinline__ int state_tile_off(int nt, int pt, int lane) {
    return ((nt * (P / 16) + pt) * 64 + lane) * 16;
}

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
    const int4 *chunks;       // {seq, chunk index in seq, first token, length | kLastChunk on a sequence's last}
    const int *n_chunks;      // number of valid chunk entries
    int *tickets;             // one counter per XCD
    const int *items;         // per-XCD work-item lists, concatenated
    const int *xcd_count;     // items per XCD
    const int *xcd_offset;    // start of each XCD's list
    int n_xcd;
    int *flags;               // per (sequence, head): published state parts (kWaves per chunk)
    int flag_stride;          // ints between consecutive flags (one cache line apart, or packed)
    int *error;
    // H counts kernel heads of P channels.  A head dim wider than the kernel
    // tile (P = 128 on 64-wide tiles) runs as `hsub` consecutive kernel heads
    // per model head: x, y and the states are then exactly the layout of
    // H = hsub * nheads heads of P channels (every state row depends only on
    // its own channel of x and on the head's shared dt, A, B, C), while dt, A,
    // D and dt_bias are indexed by the model head h / hsub.
    int H, G;
    int hsub;                 // kernel heads per model head (1 or 2)
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
    static constexpr int BLK = 64;               // tokens per decay block
    static constexpr int KPB = BLK / 32;         // K steps per decay block
    static constexpr int TPB = BLK / 16;         // 16-row tiles per decay block
    static constexpr int NBLK = Q / BLK;
    static constexpr bool kTwoTiles = QT > kWaves;   // waves own tiles w and 2*kWaves-1-w
    static constexpr int GT = kTwoTiles ? QT + 1 : QT; // C B^T tiles held per wave
    // chunk-state work split: WN waves along the state dim, WP along the head dim
    static constexpr int WN = cmin(NT, kWaves);
    static constexpr int WP = kWaves / WN;
    static constexpr int NTW = (NT + WN - 1) / WN;   // state tiles per wave
    static constexpr int PTW = (PT + WP - 1) / WP;   // head-dim tiles per wave
    static constexpr int E = (int)sizeof(IO);
    static constexpr int FRAG_REGS = 8 * E / 4;  // registers per MFMA operand fragment
    // bf16 tiles are unpadded and swizzled (lds_off); fp32 rows carry 16 bytes of padding
    static constexpr int PAD = E == 2 ? 0 : 16 / E;
    static constexpr int SB = NP + PAD;          // row stride of the B chunk
    static constexpr int SX = Q + PAD;           // row stride of the x^T tiles
    static constexpr int SH = NP + PAD;          // row stride of the incoming state
    static constexpr int kLdsB = Q * SB * E;
    static constexpr int kLdsX = P * SX * E;
    static constexpr int kLdsH = P * SH * E;
    static constexpr int kNVec = 6;              // per-token float vectors (+ dt/A staging)
    static constexpr int kLdsVec = kNVec * Q * 4 + 32;
    static constexpr int kLdsMax = 160 * 1024;
    // B^T operands of the chunk state kept in registers across the heads of an
    // item; B is then read from LDS only while the item is set up.
    static constexpr bool kBtRegs = NTW * QK * FRAG_REGS <= 32;
    // (the C-in-LDS read-out below needs the B chunk's space to itself)
    // LDS: [vectors][x^T][xh^T][incoming state][B chunk].  Where that does not
    // fit, the state tile shares xh^T's space (xh^T is dead once the compute
    // phase has ended) and/or the B chunk shares the per-head tiles' space
    // (it is dead once an item is set up, when its B^T operands are in
    // registers).
    static constexpr int kHeadSep = 2 * kLdsX + kLdsH;
    static constexpr bool kCInLdsWanted = kBtRegs;
    static constexpr int kHeadAl = 2 * kLdsX > kLdsX + kLdsH ? 2 * kLdsX : kLdsX + kLdsH;
    static constexpr bool kFitSep = kLdsVec + kHeadSep + kLdsB <= kLdsMax;
    static constexpr bool kFitAliasH = kLdsVec + kHeadAl + kLdsB <= kLdsMax;
    static constexpr bool kFitAliasB = kBtRegs && kLdsVec + cmax(kHeadSep, kLdsB) <= kLdsMax;
    static constexpr bool kFitAliasHB = kBtRegs && kLdsVec + cmax(kHeadAl, kLdsB) <= kLdsMax;
    static constexpr bool kAliasB = !kFitSep && !kFitAliasH && (kFitAliasB || kFitAliasHB);
    static constexpr bool kAliasH = !kFitSep && (kFitAliasH ? true : !kFitAliasB);
    static constexpr int kHeadBytes = kAliasH ? kHeadAl : kHeadSep;
    static constexpr int kOffX = kLdsVec;
    static constexpr int kOffXh = kOffX + kLdsX;
    static constexpr int kOffH = kAliasH ? kOffXh : kOffXh + kLdsX;
    static constexpr int kOffB = kAliasB ? kOffX : kOffX + kHeadBytes;
    static constexpr int kLds = kAliasB ? kLdsVec + cmax(kHeadBytes, kLdsB) : kLdsVec + kHeadBytes + kLdsB;
    // C rows for the read-out in the B chunk's LDS (dead once B^T is in registers)
    static constexpr bool kCInLds = kCInLdsWanted && !kAliasB;
    // y rows leave through LDS (xh^T's space, of exactly the y tile's size) when
    // they are 128 bytes (bf16, P = 64) and that space is not the state tile's
    static constexpr bool kYViaLds = E == 2 && P == 64 && !kAliasH;
    static constexpr bool kFits = (kFitSep || kFitAliasH || kFitAliasB || kFitAliasHB) && QT <= 2 * kWaves &&
                                  Q % BLK == 0;
};

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

// Element offset of (row, col) in an LDS tile of COLS columns.  bf16 tiles
// are stored unpadded, with the 16-byte chunk index of each element (col / 8)
// XORed with the low bits of its row.  A fragment read (16 rows, 16 bytes per
// lane, the four lane groups at four consecutive chunks) then hands each run
// of 8 lanes one half of the 64 banks, the other half going to the run it is
// served with, where a plain row-major layout put two lanes of such a pair on
// the same banks.  fp32 tiles keep 16 bytes of padding per row instead.  COLS
// is a power of two of at least 32 in every built shape, so the XOR stays
// inside the row, and a 4- or 8-element group at a multiple of its size keeps
// its elements together and in order.
template <typename IO, int COLS>
__device__ __forceinline__ int lds_off(int row, int col) {
    if constexpr (sizeof(IO) == 2) {
        static_assert((COLS & (COLS - 1)) == 0 && COLS >= 32, "swizzled rows need a power-of-two width");
        constexpr int CH = COLS / 8;
        constexpr int MASK = (CH < 16 ? CH : 16) - 1;
        return row * COLS + (col ^ ((row & MASK) << 3));
    } else {
        return row * (COLS + 16 / (int)sizeof(IO)) + col;
    }
}

constexpr int kPastEnd = 0x40000000;   // a byte offset beyond every buffer of the kernel

// s_waitcnt operand that waits until at most n vector memory operations are
// outstanding (and for nothing else): vmcnt in bits 3:0 and 15:14, expcnt (7)
// and lgkmcnt (15) at their no-wait maxima.
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <typename IO, int AUX = 0>
__device__ __forceinline__ typename Io<IO>::Frag buf_load_frag(__amdgpu_buffer_rsrc_t r, int off) {
    typedef typename Io<IO>::Frag Frag;
    if constexpr (sizeof(IO) == 2) {
        return __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
    } else {
        const i32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
        const i32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, AUX);
        return __builtin_bit_cast(Frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
}

template <typename IO>
__device__ __forceinline__ void buf_store_half(typename Io<IO>::Half v, __amdgpu_buffer_rsrc_t r, int off) {
    if constexpr (sizeof(IO) == 2) {
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, v), r, off, 0, 0);
    } else {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, off, 0, 0);
    }
}

template <int AUX = 0>
__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX));
}

// Element offset of (row = channel, col = K-slot position) in the x^T and xh^T
// tiles: lds_off's swizzle with bits 4-5 of the row also XORed into chunk bits
// 1-2.  A fragment read (rows 16 pt .. 16 pt + 15) sees lds_off's pattern
// XORed with a constant; the staging writes (eight channel blocks of one token
// group per 8-lane run, see Prefetch) then land on distinct banks as well.
template <typename IO, int COLS>
__device__ __forceinline__ int x_lds_off(int row, int col) {
    if constexpr (sizeof(IO) == 2) {
        constexpr int CH = COLS / 8;
        constexpr int MASK = (CH < 16 ? CH : 16) - 1;
        return row * COLS + (col ^ (((row ^ ((row >> 4) << 1)) & MASK) << 3));
    } else {
        return lds_off<IO, COLS>(row, col);
    }
}

// Element offset of (row, col) in the y tile staged for the output stores:
// rows of 64 bf16 (128 bytes), the 16-byte chunk index XORed with bits 1..3 of
// the row, so that sixteen lanes writing 8 bytes at one column of sixteen rows,
// and eight lanes reading one row's eight chunks, spread over the banks.
__device__ __forceinline__ int y_lds_off(int row, int col) { return row * 64 + (col ^ (((row >> 1) & 7) << 3)); }

// Unscaled B^T fragment in the K-slot order above: lane holds
// B[k0 + 16 * (e / 4) + 4 * lg + e % 4][n0 + li], e = 0..7.
template <typename IO, int NP>
__device__ __forceinline__ typename Io<IO>::Frag load_bt_frag(const IO *sB, int k0, int n0, int li, int lg) {
    typename Io<IO>::Frag f;
    if constexpr (sizeof(IO) == 2) {
        const int row = k0 + 4 * lg + (li >> 2);
        const int col = n0 + 4 * (li & 3);
        const bf16x4 lo = lds_read_tr16(reinterpret_cast<const bf16 *>(sB + lds_off<IO, NP>(row, col)));
        const bf16x4 hi = lds_read_tr16(reinterpret_cast<const bf16 *>(sB + lds_off<IO, NP>(row + 16, col)));
        f = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = sB[lds_off<IO, NP>(k0 + 16 * (e >> 2) + 4 * lg + (e & 3), n0 + li)];
    }
    return f;
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
    // vector memory operations issued by load()
    static constexpr int kLoads = NU * 4 * (sizeof(IO) == 2 ? 1 : 2) + R + 3;
    static_assert(kLoads < 64, "vmcnt holds at most 63");
    Frag x[NU][4];
    float dt[R];
    float a;   // A[h] (wave 0)
    float d;   // D[h], 0 without D (wave 0)
    float braw; // dt_bias[h] (A[h] when there is no bias; not used then)

    // Unit u covers tokens 4*t4 .. 4*t4+3 and channels p0 .. p0+7.  With 64
    // channels (eight blocks), the eight lanes of a run take the eight blocks
    // of one token group, so a wave's load instruction reads whole 128-byte
    // rows of x (non-temporal: each row is read once); lane bit 3 and lane
    // bits 4-5 pick the token group, which with x_lds_off's swizzle keeps the
    // 8-byte staging writes of 32 lanes on distinct banks.  Other widths: sixteen consecutive units take sixteen
    // consecutive token groups of one channel block.
    static __device__ __forceinline__ int unit_t4(int u) {
        if constexpr (PB == 8) return 8 * (u >> 6) + 4 * ((u >> 3) & 1) + ((u >> 4) & 3);
        else return (u & 15) + 16 * (u / (16 * PB));
    }
    static __device__ __forceinline__ int unit_p0(int u) {
        if constexpr (PB == 8) return 8 * (u & 7);
        else return ((u >> 4) % PB) * 8;
    }

    // Head h's x chunk (every wave) and its dt, A, D and dt_bias (wave 0;
    // empty buffers elsewhere); tokens past the chunk read 0.  `live` false
    // (no such head) empties every buffer, so the same loads are issued.
    __device__ __forceinline__ void load(const FwdParams &prm, long long tok0, int q, int h, int tid, int wave,
                                         bool live) {
        const int xs = prm.H * P;
        const IO *xg = reinterpret_cast<const IO *>(prm.x) + tok0 * xs + h * P;
        const __amdgpu_buffer_rsrc_t rx = buf_rsrc(xg, live ? q * xs * S::E : 0);
#pragma unroll
        for (int k = 0; k < NU; ++k) {
            const int u = tid + k * S::kThreads;
            const int t4 = unit_t4(u);
            const int p0 = unit_p0(u);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int i = 4 * t4 + t;   // i >= q lies past the buffer's end
                const bool uok = NUNIT % S::kThreads == 0 || u < NUNIT;
                x[k][t] = buf_load_frag<IO, PB == 8 ? kStream : 0>(rx, uok ? (i * xs + p0) * S::E : kPastEnd);
            }
        }
        const int hm = h / prm.hsub, Hm = prm.H / prm.hsub;
        const bool mine = live && wave == 0;
        const __amdgpu_buffer_rsrc_t rdt = buf_rsrc(prm.dt + tok0 * Hm + hm, mine ? ((q - 1) * Hm + 1) * 4 : 0);
        const int lane = tid & 63;
#pragma unroll
        for (int k = 0; k < R; ++k) dt[k] = buf_load_f32(rdt, (lane * R + k) * Hm * 4);
        a = buf_load_f32(buf_rsrc(prm.A + hm, mine ? 4 : 0), 0);
        d = buf_load_f32(buf_rsrc(prm.D ? prm.D + hm : prm.A, mine && prm.D ? 4 : 0), 0);
        braw = buf_load_f32(buf_rsrc((prm.dtp.bias ? prm.dtp.bias : prm.A) + hm, mine ? 4 : 0), 0);
    }

    // wave 0: dt (lane holds tokens R*lane .. R*lane+R-1, preprocessed when
    // asked; tokens past the chunk stay 0), A and D into LDS
    __device__ __forceinline__ void stage_dt(float *sStage, int lane, int q, const DtProc &dtp) const {
#pragma unroll
        for (int k = 0; k < R; ++k) {
            float v = dt[k];
            if (dtp.on && lane * R + k < q) v = dtp.apply(v, dtp.bias ? braw : 0.f);
            sStage[lane * R + k] = v;
        }
        if (lane == 0) {
            sStage[Q] = a;
            sStage[Q + 1] = d;
        }
    }

    // x^T[p][i .. i+3] from 4 tokens of one channel, as is into sX and times
    // the per-token factor into sXh.  fh(k) holds the factor of the scan
    // lane's k-th token (R consecutive tokens per lane of the wave).
    template <typename FH>
    __device__ __forceinline__ void stage(IO *sX, IO *sXh, int tid, FH fh) const {
        typedef typename Io<IO>::Half Half;
#pragma unroll
        for (int k = 0; k < NU; ++k) {
            const int u = tid + k * S::kThreads;
            const int t4 = unit_t4(u);
            const int p0 = unit_p0(u);
            float fac[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) fac[t] = fh(t % R, (4 * t4 + t) / R);   // every lane shuffles
            if (u < NUNIT) {
                const int pos = xpos(4 * t4);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    Half v, w;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        v[t] = x[k][t][e];
                        w[t] = from_f32<IO>(to_f32(x[k][t][e]) * fac[t]);
                    }
                    *reinterpret_cast<Half *>(sX + x_lds_off<IO, Q>(p0 + e, pos)) = v;
                    *reinterpret_cast<Half *>(sXh + x_lds_off<IO, Q>(p0 + e, pos)) = w;
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
    IO *sX = reinterpret_cast<IO *>(smem + S::kOffX);
    IO *sXh = reinterpret_cast<IO *>(smem + S::kOffXh);
    IO *sH = reinterpret_cast<IO *>(smem + S::kOffH);
    IO *sB = reinterpret_cast<IO *>(smem + S::kOffB);
    float *vDt = vS2 + Q;     // dt_j
    float *vCol = vDt + Q;    // exp(s_r - s_j) dt_j, r = last token of j's 16-tile
    float *vEo = vCol + Q;    // exp(s_i)
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
        const int q = ce.w & (kLastChunk - 1);
        const bool last = (ce.w & kLastChunk) != 0;
        const int xs = H * P;          // token stride of x and y (elements)
        const int bs = G * N;          // token stride of B and C
        const IO *Bg = reinterpret_cast<const IO *>(prm.B) + tok0 * bs + g * N;
        const IO *Cg = reinterpret_cast<const IO *>(prm.C) + tok0 * bs + g * N;

        // ---- every global load of the item's set-up, issued together ----
        // The first head's x and dt, the chunk's B rows and the C rows of
        // this wave's tiles (which, over the eight waves, are every row of the
        // chunk: they also fill the C tile of the read-out), as branch-free
        // buffer loads (rows past the chunk lie past the buffers' end and read
        // 0): one memory round trip, and each group is waited for only where
        // it is used.
        Prefetch<IO, P, N, Q> pf;
        pf.load(prm, tok0, q, h_begin, tid, wave, true);
        constexpr int VPR = S::NP * S::E / 16;   // 16-byte vectors per padded row
        constexpr int VN = N * S::E / 16;        // vectors that hold data
        constexpr int NV = (Q * VPR + S::kThreads - 1) / S::kThreads;
        const int rows_bytes = q > 0 ? ((q - 1) * bs + N) * S::E : 0;
        const __amdgpu_buffer_rsrc_t rB = buf_rsrc(Bg, rows_bytes);
        const __amdgpu_buffer_rsrc_t rC = buf_rsrc(Cg, rows_bytes);
        auto row_vec = [&](int k, int &j, int &c) {   // vector k of this thread: row j, 16-byte column c
            const int u = tid + k * S::kThreads;
            j = u / VPR;
            c = u - j * VPR;
            return (Q * VPR % S::kThreads == 0 || u < Q * VPR);
        };
        auto row_vec_off = [&](int k) {
            int j, c;
            const bool ok = row_vec(k, j, c) && c < VN;
            return ok ? (j * bs + c * (16 / S::E)) * S::E : kPastEnd;
        };
        i32x4 bv[NV];
    #pragma unroll
        for (int k = 0; k < NV; ++k) bv[k] = __builtin_amdgcn_raw_buffer_load_b128(rB, row_vec_off(k), 0, 0);

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
                cf[ks] = buf_load_frag<IO>(rC, n0 < N ? ((16 * I + li) * bs + n0) * S::E : kPastEnd);
            }
        };
        Frag cga[S::NK], cgb[S::NK];
        load_c(hasA ? Ia : S::QT, cga);
        load_c(hasB ? Ib : S::QT, cgb);
        // the B rows into LDS
    #pragma unroll
        for (int k = 0; k < NV; ++k) {
            int j, c;
            if (row_vec(k, j, c)) *reinterpret_cast<i32x4 *>(sB + lds_off<IO, S::NP>(j, c * (16 / S::E))) = bv[k];
        }
        if (wave == 0) pf.stage_dt(sStage, lane, q, prm.dtp);
        __syncthreads();  // B chunk and the first head's dt in LDS
        // Runs f with this wave's index as a compile-time constant, so that the
        // phases below are unrolled without any branch on the wave's row tiles.
        auto with_wave = [&](auto f) {
            static_assert(S::kWaves == 8, "one case per wave");
            switch (wave) {
            case 0: f(std::integral_constant<int, 0>{}); break;
            case 1: f(std::integral_constant<int, 1>{}); break;
            case 2: f(std::integral_constant<int, 2>{}); break;
            case 3: f(std::integral_constant<int, 3>{}); break;
            case 4: f(std::integral_constant<int, 4>{}); break;
            case 5: f(std::integral_constant<int, 5>{}); break;
            case 6: f(std::integral_constant<int, 6>{}); break;
            default: f(std::integral_constant<int, 7>{}); break;
            }
        };
        // Kept in the io precision (the MFMAs take them in it); fp32 accumulation.
        // Tile (Ia, J) for J <= Ia, else (Ib, GT-1-J); rows past the chunk hold
        // zeros in B and C, so their tiles come out 0 without a test.  The K
        // loop is outermost, so the tiles' independent MFMA chains interleave.
        Half gtile[S::GT];
        with_wave([&](auto wc) {
            constexpr int W = decltype(wc)::value;
            f32x4 acc[S::GT];
    #pragma unroll
            for (int J = 0; J < S::GT; ++J) acc[J] = zero4();
    #pragma unroll
            for (int ks = 0; ks < S::NK; ++ks) {
    #pragma unroll
                for (int J = 0; J < S::GT; ++J) {
                    const bool useA = J <= W;
                    const bool live = useA ? W < S::QT : S::kTwoTiles;
                    const int jt = useA ? J : S::GT - 1 - J;
                    if (live) {
                        const Frag bfr = *reinterpret_cast<const Frag *>(sB + lds_off<IO, S::NP>(16 * jt + li, ks * 32 + 8 * lg));
                        acc[J] = Io<IO>::mfma(acc[J], bfr, useA ? cga[ks] : cgb[ks]);
                    }
                }
            }
    #pragma unroll
            for (int J = 0; J < S::GT; ++J)
    #pragma unroll
                for (int r = 0; r < 4; ++r) gtile[J][r] = from_f32<IO>(acc[J][r]);
        });

        const int wn = wave % S::WN;
        const int wp = wave / S::WN;
        // B^T operands of the chunk state for this wave's state tiles, all K steps
        Frag btr[S::kBtRegs ? S::NTW : 1][S::kBtRegs ? S::QK : 1];
        if constexpr (S::kBtRegs) {
    #pragma unroll
            for (int a = 0; a < S::NTW; ++a) {
                const int nt = wn + a * S::WN;
    #pragma unroll
                for (int ks = 0; ks < S::QK; ++ks) {
                    btr[a][ks] = zero_frag<Frag>();
                    if (wp < S::PT && nt < S::NT) btr[a][ks] = load_bt_frag<IO, S::NP>(sB, ks * 32, nt * 16, li, lg);
                }
            }
        }
        // With the B^T operands in registers, the B chunk is dead: its LDS then
        // holds the chunk's C rows for the read-out (row layout, like B),
        // written from the C fragments of the waves' row tiles (tiles w and
        // 2 kWaves - 1 - w cover the chunk; rows past it hold zeros).
        IO *sC = sB;
        if constexpr (S::kBtRegs) {
            __syncthreads();   // every wave is done with the B chunk
            if constexpr (S::kCInLds) {
    #pragma unroll
                for (int ks = 0; ks < S::NK; ++ks) {
                    const int col = ks * 32 + 8 * lg;
                    if (Ia < S::QT) *reinterpret_cast<Frag *>(sC + lds_off<IO, S::NP>(16 * Ia + li, col)) = cga[ks];
                    if (S::kTwoTiles) *reinterpret_cast<Frag *>(sC + lds_off<IO, S::NP>(16 * Ib + li, col)) = cgb[ks];
                }
            }
            // (read only after the first head's staging barrier)
        } else if constexpr (S::kAliasB) {
            __syncthreads();   // the per-head tiles overwrite the B chunk
        }

        // C B^T fragment (rows of tile I, K step ks) straight from the
        // registers, for the blocks left of the row's own decay block.
        auto cb_frag = [&](auto from_a, int ks) {
            constexpr bool fromA = decltype(from_a)::value;
            Frag m;
    #pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int jt = 2 * ks + half;
                const Half &gh = gtile[fromA ? jt : S::GT - 1 - jt];
    #pragma unroll
                for (int r = 0; r < 4; ++r) m[4 * half + r] = gh[r];
            }
            return m;
        };
        // Decay-weighted mask fragment of tile I, K step ks, inside the row's
        // own decay block: lane holds M[i_row][j], j = 32 ks + 16 half + 4 lg + r.
        // Below the diagonal 16-tile: G * exp(s_i - s_r) * exp(s_r - s_j) dt_j
        // (both factors <= 1, r the last token of j's 16-tile); on it the exact
        // exp(s_i - s_j) with a causal select, and the skip coefficient D added
        // on the diagonal itself (y_i gains D x_i from the same product).
        auto mask_frag = [&](auto from_a, int I, int ks, float s2_i, const float (&sref)[S::QT], float dh) {
            constexpr bool fromA = decltype(from_a)::value;
            const int i_row = 16 * I + li;
            Frag m;
    #pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int jt = 2 * ks + half;
                const int j0 = 32 * ks + 16 * half + 4 * lg;
                const Half &gh = gtile[fromA ? jt : S::GT - 1 - jt];   // C B^T tile (I, jt)
                f32x4 gv;
    #pragma unroll
                for (int r = 0; r < 4; ++r) gv[r] = to_f32(gh[r]);
                if (jt < I) {
                    const float rowf = exp2f_fast(s2_i - sref[jt]);
                    const f32x4 colv = *reinterpret_cast<const f32x4 *>(vCol + j0);
    #pragma unroll
                    for (int r = 0; r < 4; ++r) m[4 * half + r] = from_f32<IO>(gv[r] * rowf * colv[r]);
                } else if (jt == I) {
                    const f32x4 s2j = *reinterpret_cast<const f32x4 *>(vS2 + j0);
                    const f32x4 dtj = *reinterpret_cast<const f32x4 *>(vDt + j0);
    #pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float v = gv[r] * exp2f_fast(s2_i - s2j[r]) * dtj[r] + (j0 + r == i_row ? dh : 0.f);
                        m[4 * half + r] = from_f32<IO>((j0 + r <= i_row) ? v : 0.f);
                    }
                } else {
    #pragma unroll
                    for (int r = 0; r < 4; ++r) m[4 * half + r] = from_f32<IO>(0.f);
                }
            }
            return m;
        };
        // Row tiles of wave W: tile a = W, tile b = 2 kWaves - 1 - W (chunks of
        // 2 kWaves tiles); each tile's decay block R, and its explicit K steps
        // [KPB R, I / 2] (the steps before them run on the C B^T tiles as is).
        struct WaveTiles {
            int IA, IB, RA, RB, EA0, EA1, EB0, EB1;
            bool HA, HB;
        };
        auto tiles_of = [](auto wc) {
            constexpr int W = decltype(wc)::value;
            WaveTiles t{};
            t.IA = W;
            t.IB = 2 * S::kWaves - 1 - W;
            t.HA = W < S::QT;
            t.HB = S::kTwoTiles;
            t.RA = t.IA / S::TPB;
            t.RB = t.IB / S::TPB;
            t.EA0 = S::KPB * t.RA;
            t.EA1 = t.IA / 2;
            t.EB0 = S::KPB * t.RB;
            t.EB1 = t.IB / 2;
            return t;
        };

        int *sReady = sTicket + 1;
        // Cache policy of the hand-off: the stores are ordinary, so H_{c+1}
        // stays in this XCD's L2 (write-back); the loads (state and counter)
        // are device scope (sc1), which skips the compute unit's L1 (it may
        // hold an older version of these in-place lines) and is served by the
        // same L2.
        constexpr int kStateLoad = 16;   // sc1

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

            // ---- (1) in-chunk cumulative sum, per-token vectors, x^T and xh^T ----
            float Dh;   // skip coefficient D[h] (0 without D)
            {
                // one early look at the predecessor's flag (the state loads can
                // then be issued before the compute phase)
                // (compared only after the scan, so that the scan does not wait for it)
                // (wave 0 reads it; an empty buffer elsewhere and for the first chunk)
                int flagv = __builtin_bit_cast(
                    int, buf_load_f32<kStateLoad>(buf_rsrc(prm.flags + (long long)unit * prm.flag_stride, wave == 0 && cloc > 0 ? 4 : 0), 0));
                // Every wave scans the whole chunk (R tokens per lane, from the
                // staged dt) and writes the per-token vectors of its own Q/8
                // tokens (lanes 8 wave .. 8 wave + 7).
                constexpr int R = Q / 64;
                const float Ah = sStage[Q];
                Dh = sStage[Q + 1];
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
                // last token of each 16-token tile: index (i | 15), held by lane ((i | 15) / R);
                // likewise the last token of each 64-token decay block
                const float ref = __shfl(s2[R - 1], ((lane * R) | 15) / R, 64);
                const float ref64 = __shfl(s2[R - 1], ((lane * R) | (S::BLK - 1)) / R, 64);
                float fh[R];   // staging factor of xh: exp(e_b - s_j) dt_j
    #pragma unroll
                for (int k = 0; k < R; ++k) fh[k] = exp2f_fast(ref64 - s2[k]) * dtv[k];
                if ((lane >> 3) == wave) {
    #pragma unroll
                    for (int k = 0; k < R; ++k) {
                        const int i = lane * R + k;
                        const float d = dtv[k];
                        vS2[i] = s2[k];
                        vDt[i] = d;
                        vCol[i] = exp2f_fast(ref - s2[k]) * d;
                        vEo[i] = exp2f_fast(s2[k]);
                        if ((i & 15) == 15) vRef[i >> 4] = s2[k];
                    }
                }
                pf.stage(sX, sXh, tid, [&](int k, int src) { return __shfl(fh[k], src, 64); });
                asm volatile("" : "+v"(flagv));   // keeps the comparison (and its wait) here
                if (wave == 0 && lane == 0) *sReady = cloc == 0 || flagv >= S::kWaves * cloc;
            }
            __syncthreads();
            const float s2_last = vS2[Q - 1];
            const bool early = *sReady != 0;

            // Incoming boundary state: issued here, ahead of the compute phase,
            // when the predecessor had already published (its latency then
            // hides behind the compute phase), else after the wait below.
            const float *hin = (cloc == 0) ? (prm.init_state ? prm.init_state + (long long)unit * P * N : nullptr)
                                           : prm.state + (long long)unit * P * N;
            float *hout = prm.state + (long long)unit * P * N;
            f32x4 hv[S::NTW][S::PTW];
            auto load_state = [&](bool on) {   // (off: an empty buffer, the same loads)
                const __amdgpu_buffer_rsrc_t rin = buf_rsrc(hin, hin && on ? P * N * 4 : 0);
    #pragma unroll
                for (int a = 0; a < S::NTW; ++a)
    #pragma unroll
                    for (int b = 0; b < S::PTW; ++b) {
                        const int nt = wn + a * S::WN, pt = wp + b * S::WP;
                        const bool ok = wp < S::PT && nt < S::NT && pt < S::PT;
                        hv[a][b] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                            rin, !ok ? kPastEnd : cloc == 0 ? ((pt * 16 + li) * N + nt * 16 + 4 * lg) * 4
                                                            : state_tile_off<P>(nt, pt, li + 16 * lg), 0, kStateLoad));
                    }
            };
            load_state(early);

            // ---- (2) compute: chunk state and both tiles' diagonal blocks ----
            // One pass over the K steps.  Each step reads the xh^T fragments of
            // every head-dim tile once, for the chunk state and for the rows whose
            // decay block lies right of the step; rows inside their own block
            // take the x^T fragments and the explicit mask instead.  The next
            // step's xh^T (and B^T) fragments are read while the current step's
            // MFMAs run (the scheduling barriers keep that order).
            // S_c^T = B^T xh: accumulator element r of tile (nt, pt) is S_c[p][n]
            // with p = pt*16 + li and n = nt*16 + 4*lg + r.  Diagonal blocks are
            // computed transposed (Y^T = x^T M^T): element r of tile pt is
            // Y_diag[16 I + li][pt*16 + 4*lg + r].
            float sref[S::QT];   // 16-tile reference cumsums, wave-uniform
    #pragma unroll
            for (int t = 0; t < S::QT; ++t)
                sref[t] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, vRef[t])));
            f32x4 accS[S::NTW][S::PTW];
    #pragma unroll
            for (int a = 0; a < S::NTW; ++a)
    #pragma unroll
                for (int b = 0; b < S::PTW; ++b) accS[a][b] = zero4();
            f32x4 accYa[S::PT], accYb[S::PT];
    #pragma unroll
            for (int pt = 0; pt < S::PT; ++pt) {
                accYa[pt] = zero4();
                accYb[pt] = zero4();
            }
            auto scale4 = [](f32x4 (&acc)[S::PT], float f) {
    #pragma unroll
                for (int pt = 0; pt < S::PT; ++pt)
    #pragma unroll
                    for (int r = 0; r < 4; ++r) acc[pt][r] *= f;
            };
            with_wave([&](auto wc) {
                constexpr int W = decltype(wc)::value;
                constexpr WaveTiles T = tiles_of(wc);
                constexpr int WNc = W % S::WN, WPc = W / S::WN;
                constexpr bool HS = WPc < S::PT;   // the wave has chunk-state tiles
                const float s2_ia = T.HA ? vS2[16 * T.IA + li] : 0.f;
                const float s2_ib = T.HB ? vS2[16 * T.IB + li] : 0.f;
                Frag xh[2][S::PT];
                Frag bt[2][S::NTW];
                auto load_step = [&](int ks, Frag (&xo)[S::PT], Frag (&bo)[S::NTW]) {
    #pragma unroll
                    for (int pt = 0; pt < S::PT; ++pt)
                        xo[pt] = *reinterpret_cast<const Frag *>(sXh + x_lds_off<IO, Q>(pt * 16 + li, ks * 32 + 8 * lg));
    #pragma unroll
                    for (int a = 0; a < S::NTW; ++a) {
                        const int nt = WNc + a * S::WN;
                        if constexpr (S::kBtRegs) bo[a] = btr[a][ks];
                        else bo[a] = (HS && nt < S::NT) ? load_bt_frag<IO, S::NP>(sB, ks * 32, nt * 16, li, lg)
                                                        : zero_frag<Frag>();
                    }
                };
                load_step(0, xh[0], bt[0]);
    #pragma unroll
                for (int ks = 0; ks < S::QK; ++ks) {
                    const int cur = ks & 1;
                    const int blk = ks / S::KPB;
                    if (ks + 1 < S::QK) load_step(ks + 1, xh[cur ^ 1], bt[cur ^ 1]);
                    __builtin_amdgcn_sched_barrier(0);
                    // x^T fragments of the rows whose own block this step is in
                    const bool exA = T.HA && ks >= T.EA0 && ks <= T.EA1;
                    const bool exB = T.HB && ks >= T.EB0 && ks <= T.EB1;
                    Frag xea[S::PT], xeb[S::PT];
    #pragma unroll
                    for (int pt = 0; pt < S::PT; ++pt) {
                        if (exA) xea[pt] = *reinterpret_cast<const Frag *>(sX + x_lds_off<IO, Q>(pt * 16 + li, ks * 32 + 8 * lg));
                        if (exB) xeb[pt] = *reinterpret_cast<const Frag *>(sX + x_lds_off<IO, Q>(pt * 16 + li, ks * 32 + 8 * lg));
                    }
                    if (ks % S::KPB == 0 && blk > 0) {
                        // block decay exp(e_b - e_{b-1}) on every sum still in its recurrence
                        const float dl = exp2f_fast(sref[S::TPB * blk + S::TPB - 1] - sref[S::TPB * blk - 1]);
    #pragma unroll
                        for (int a = 0; a < S::NTW; ++a)
    #pragma unroll
                            for (int b = 0; b < S::PTW; ++b)
    #pragma unroll
                                for (int r = 0; r < 4; ++r) accS[a][b][r] *= dl;
                        if (T.HA && blk < T.RA) scale4(accYa, dl);
                        if (T.HB && blk < T.RB) scale4(accYb, dl);
                    }
                    // entering the row's own block: the row factor exp(s_i - e_{R-1})
                    if (T.HA && T.RA > 0 && ks == T.EA0) scale4(accYa, exp2f_fast(s2_ia - sref[S::TPB * T.RA - 1]));
                    if (T.HB && T.RB > 0 && ks == T.EB0) scale4(accYb, exp2f_fast(s2_ib - sref[S::TPB * T.RB - 1]));
                    if (HS) {
    #pragma unroll
                        for (int a = 0; a < S::NTW; ++a)
    #pragma unroll
                            for (int b = 0; b < S::PTW; ++b) {
                                const int pt = WPc + b * S::WP;
                                if (WNc + a * S::WN < S::NT && pt < S::PT)
                                    accS[a][b] = Io<IO>::mfma(accS[a][b], bt[cur][a], xh[cur][pt]);
                            }
                    }
                    if (T.HA && ks < T.EA0) {
                        const Frag m = cb_frag(std::true_type{}, ks);
    #pragma unroll
                        for (int pt = 0; pt < S::PT; ++pt) accYa[pt] = Io<IO>::mfma(accYa[pt], xh[cur][pt], m);
                    }
                    if (T.HB && ks < T.EB0) {
                        const Frag m = cb_frag(std::false_type{}, ks);
    #pragma unroll
                        for (int pt = 0; pt < S::PT; ++pt) accYb[pt] = Io<IO>::mfma(accYb[pt], xh[cur][pt], m);
                    }
                    if (exA) {
                        const Frag m = mask_frag(std::true_type{}, T.IA, ks, s2_ia, sref, Dh);
    #pragma unroll
                        for (int pt = 0; pt < S::PT; ++pt) accYa[pt] = Io<IO>::mfma(accYa[pt], xea[pt], m);
                    }
                    if (exB) {
                        const Frag m = mask_frag(std::false_type{}, T.IB, ks, s2_ib, sref, Dh);
    #pragma unroll
                        for (int pt = 0; pt < S::PT; ++pt) accYb[pt] = Io<IO>::mfma(accYb[pt], xeb[pt], m);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            });

            // ---- (3) chain: wait if needed, H_{c+1} = exp(s_last) H_c + S_c, H_c to LDS ----
            // One thread waits for the predecessor's counter, then every wave
            // loads the incoming state.
            if (!early || S::kAliasH) {
                if (!early && tid == 0) {
                    int it = 0;
                    while (__hip_atomic_load(prm.flags + (long long)unit * prm.flag_stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                           S::kWaves * cloc) {
                        __builtin_amdgcn_s_sleep(1);
                        if (++it > (1 << 22)) {
                            atomicOr(prm.error, 1);
                            break;
                        }
                    }
                }
                // (also: with the state tile over xh^T, every wave has left the compute phase)
                __syncthreads();
                if (!early) load_state(true);
            }
            Frag cfa[S::kCInLds ? 1 : S::NK], cfb[S::kCInLds ? 1 : S::NK];
            if constexpr (!S::kCInLds) {
                load_c(hasA ? Ia : S::QT, cfa);
                load_c(hasB ? Ib : S::QT, cfb);
            }
            const float alpha = exp2f_fast(s2_last);
            if constexpr (SSD_RACE_WIDEN != 0) race_widen_delay(unit, cloc, wave);
            // A sequence's first and last chunks read and write the state in
            // different orders (row-major in and tile order out, or the
            // reverse), so one wave's stores could land on state that another
            // wave has yet to read (when the initial state is the output
            // buffer, or in the last chunk, always): every wave's state loads
            // complete first.  Other chunks write exactly what each wave read.
            if ((cloc == 0) != last) {
                __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
                __syncthreads();
            }
            {
                const __amdgpu_buffer_rsrc_t rout = buf_rsrc(hout, P * N * 4);
    #pragma unroll
                for (int a = 0; a < S::NTW; ++a)
    #pragma unroll
                    for (int b = 0; b < S::PTW; ++b) {
                        const int nt = wn + a * S::WN, pt = wp + b * S::WP;
                        const bool ok = wp < S::PT && nt < S::NT && pt < S::PT;
                        const int p = pt * 16 + li;
                        const int n0 = nt * 16 + 4 * lg;
                        f32x4 o;
                        Half hb;
    #pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            o[r] = alpha * hv[a][b][r] + accS[a][b][r];
                            hb[r] = from_f32<IO>(hv[a][b][r]);
                        }
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, o), rout,
                                                               !ok ? kPastEnd : last ? (p * N + n0) * 4
                                                                                    : state_tile_off<P>(nt, pt, li + 16 * lg), 0, 0);
                        if (ok) *reinterpret_cast<Half *>(sH + lds_off<IO, S::NP>(p, n0)) = hb;
                    }
            }
            // The next head's x and dt, issued after the state stores: the
            // read-out below then waits for the stores alone (vector memory
            // operations complete in issue order), and the prefetch has until
            // the next head's staging to arrive.
            __builtin_amdgcn_sched_barrier(0);
            pf.load(prm, tok0, q, h + 1, tid, wave, h + 1 < h_end);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (S::NP != N) {   // zero K slots past the state dim
                for (int v = tid; v < P * (S::NP - N); v += S::kThreads) {
                    const int p = v / (S::NP - N);
                    sH[lds_off<IO, S::NP>(p, N + (v - p * (S::NP - N)))] = from_f32<IO>(0.f);
                }
            }
            __syncthreads();  // H_c is in LDS

            // ---- (4) state read-out and outputs of both tiles ----
            // Y_off = C H_c^T for both row tiles in one pass over the state's K
            // steps (each H fragment is read once); then each wave publishes its
            // part of H_{c+1} (one increment of the (sequence, head) counter) once
            // its state stores are acknowledged -- a successor waits for all
            // kWaves increments -- and writes y = Y_diag + exp(s_i) Y_off (Y_diag
            // already holds D x, from the mask's diagonal).
            with_wave([&](auto wc) {
                constexpr WaveTiles T = tiles_of(wc);
                f32x4 oa[S::PT], ob[S::PT];
    #pragma unroll
                for (int pt = 0; pt < S::PT; ++pt) {
                    oa[pt] = zero4();
                    ob[pt] = zero4();
                }
                Frag hf[2][S::PT];
                Frag ca[2], cb[2];
                auto load_h = [&](int ks, Frag (&o)[S::PT], Frag &oa_, Frag &ob_) {
    #pragma unroll
                    for (int pt = 0; pt < S::PT; ++pt)
                        o[pt] = *reinterpret_cast<const Frag *>(sH + lds_off<IO, S::NP>(pt * 16 + li, ks * 32 + 8 * lg));
                    if constexpr (S::kCInLds) {
                        if (T.HA) oa_ = *reinterpret_cast<const Frag *>(sC + lds_off<IO, S::NP>(16 * T.IA + li, ks * 32 + 8 * lg));
                        if (T.HB) ob_ = *reinterpret_cast<const Frag *>(sC + lds_off<IO, S::NP>(16 * T.IB + li, ks * 32 + 8 * lg));
                    } else {
                        oa_ = cfa[S::kCInLds ? 0 : ks];
                        ob_ = cfb[S::kCInLds ? 0 : ks];
                    }
                };
                if (T.HA || T.HB) load_h(0, hf[0], ca[0], cb[0]);
    #pragma unroll
                for (int ks = 0; ks < S::NK; ++ks) {
                    if (!(T.HA || T.HB)) break;
                    if (ks + 1 < S::NK) load_h(ks + 1, hf[(ks + 1) & 1], ca[(ks + 1) & 1], cb[(ks + 1) & 1]);
                    __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                    for (int pt = 0; pt < S::PT; ++pt) {
                        if (T.HA) oa[pt] = Io<IO>::mfma(oa[pt], hf[ks & 1][pt], ca[ks & 1]);
                        if (T.HB) ob[pt] = Io<IO>::mfma(ob[pt], hf[ks & 1][pt], cb[ks & 1]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                // this wave's state stores are acknowledged: everything but the
                // prefetch's loads, the last ones issued, has completed
                __builtin_amdgcn_s_waitcnt(vmcnt_only(Prefetch<IO, P, N, Q>::kLoads));
                // (lane 0 adds; the other lanes' offsets lie past the counter)
                (void)__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(1, buf_rsrc(prm.flags + (long long)unit * prm.flag_stride, 4), lane == 0 ? 0 : kPastEnd,
                                                                     0, 0);
                const __amdgpu_buffer_rsrc_t ry = buf_rsrc(yg, q * xs * S::E);   // rows i >= q lie past its end
                if constexpr (S::kYViaLds) {
                    // The wave's rows go through LDS (xh^T's space, dead since
                    // the compute phase) and leave as whole 128-byte rows, one
                    // 16-byte store per lane, rather than as 32-byte pieces of
                    // four stores, non-temporal (y is not read again).  Only
                    // this wave touches these rows.
                    IO *sY = sXh;
                    auto y_to_lds = [&](int I, const f32x4 (&o)[S::PT], const f32x4 (&accY)[S::PT]) {
                        const int i_row = 16 * I + li;
                        const float eo = vEo[i_row];
    #pragma unroll
                        for (int pt = 0; pt < S::PT; ++pt) {
                            Half yv;
    #pragma unroll
                            for (int r = 0; r < 4; ++r) yv[r] = from_f32<IO>(accY[pt][r] + eo * o[pt][r]);
                            *reinterpret_cast<Half *>(sY + y_lds_off(i_row, pt * 16 + 4 * lg)) = yv;
                        }
                    };
                    auto y_rows = [&](int I) {
    #pragma unroll
                        for (int k = 0; k < 2; ++k) {
                            const int row = 16 * I + 8 * k + (lane >> 3);
                            const int col = 8 * (lane & 7);
                            const i32x4 v = *reinterpret_cast<const i32x4 *>(sY + y_lds_off(row, col));
                            __builtin_amdgcn_raw_buffer_store_b128(v, ry, (row * xs + col) * S::E, 0, kStream);
                        }
                    };
                    if (T.HA) y_to_lds(T.IA, oa, accYa);
                    if (T.HB) y_to_lds(T.IB, ob, accYb);
                    if (T.HA) y_rows(T.IA);
                    if (T.HB) y_rows(T.IB);
                } else {
                    auto epilogue = [&](int I, const f32x4 (&o)[S::PT], const f32x4 (&accY)[S::PT]) {
                        const int i_row = 16 * I + li;
                        const float eo = vEo[i_row];
    #pragma unroll
                        for (int pt = 0; pt < S::PT; ++pt) {
                            Half yv;
    #pragma unroll
                            for (int r = 0; r < 4; ++r) yv[r] = from_f32<IO>(accY[pt][r] + eo * o[pt][r]);
                            buf_store_half<IO>(yv, ry, (i_row * xs + pt * 16 + 4 * lg) * S::E);
                        }
                    };
                    if (T.HA) epilogue(T.IA, oa, accYa);
                    if (T.HB) epilogue(T.IB, ob, accYb);
                }
            });
            if (wave == 0 && h + 1 < h_end) pf.stage_dt(sStage, lane, q, prm.dtp);   // the next head's dt and A
            __syncthreads();  // every wave is done with this head's LDS tiles
        }
    }
}

}  // namespace ssd

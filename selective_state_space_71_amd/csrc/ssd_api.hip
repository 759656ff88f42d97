// ssd_api.hip -- host side of libssd.so: argument validation, workspace
// layout, the chunk-schedule kernel, the decode kernel and the C ABI.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <utility>
#include <vector>

#include "ssd.h"
#include "ssd_device.h"
#include "ssd_fwd_kernel.h"
#include "ssd_block_kernels.h"
#include "ssd_bwd_kernels.h"

namespace ssd {
bool fwd_dispatch_bf16(int p, int n, int q, const FwdParams &prm, long long max_entries, hipStream_t st,
                       bool launch, hipError_t *err);
bool fwd_dispatch_f32(int p, int n, int q, const FwdParams &prm, long long max_entries, hipStream_t st,
                      bool launch, hipError_t *err);

// ---------------------------------------------------------------------------
// Chunk schedule.  Every (sequence, chunk index) pair becomes one entry
// {seq, chunk index in seq, first token, length}.  Entries are ordered by
// chunk index first and sequence second, so the predecessor of an entry
// (same sequence, previous chunk) always has a smaller index.  A work item
// is (entry, group, head slice); all items of one (sequence, group, slice)
// chain go to the same XCD, and each XCD's list keeps the entry order, so an
// item's predecessor is always earlier in the same list.  Dense batches (all
// sequences of one length) give each XCD a contiguous block of chains in
// (sequence, group, slice) order, so that the slices of a sequence share few
// XCDs and their B, C and dt rows are fetched by few L2s; packed batches go
// round robin over chains (their sequences differ in length, and a block of
// whole sequences would unbalance the XCDs).  The kernel also clears the
// tickets, the error word and the per-(sequence, head) progress flags, and
// writes the final state of empty packed sequences (the initial state, or
// zero).
struct PrepParams {
    const int *cu_seqlens;  // null for a dense batch
    int batch, seqlen, nseq, H, Q;
    int G, slices, n_xcd;
    int flag_stride;        // ints between consecutive progress flags
    int max_entries;        // capacity of the chunk table
    int state_elems;        // P * N
    int4 *chunks;
    int *n_chunks;
    int *tickets;           // [16] one per XCD
    int *error;
    int *flags;
    int *items;             // per-XCD item lists, concatenated
    int *xcd_count;         // [16]
    int *xcd_offset;        // [16]
    int *seq_chunk_start;   // [nseq + 1] scratch (packed batches)
    const float *init_state;
    float *final_state;
};

// Packed batch: chunk counts per sequence, their running sum, the
// chunk-index-major table and the final state of empty sequences.  The
// offsets are checked on the way (0 = cu[0] <= cu[1] <= ... <= cu[nseq] =
// seqlen, and at most max_entries chunks): offsets that break this leave an
// empty schedule (no chunk entries, so every forward workgroup exits at once
// and nothing is read or written out of bounds) and set bit 1 of the error
// word.  Returns false in that case.
__device__ bool build_packed_schedule(const PrepParams &p) {
    const int tid = threadIdx.x;
    const int Q = p.Q;
    const int n = p.nseq;
    // Offsets and chunk starts of up to kCache sequences are read from LDS
    // (the loops below would otherwise wait on one global load per step).
    constexpr int kCache = 4096;
    __shared__ int s_cu[kCache + 1], s_cs[kCache + 1];
    __shared__ long long s_part[256];
    __shared__ int s_bad;
    const bool cached = n <= kCache;
    if (tid == 0) s_bad = 0;
    if (cached)
        for (int i = tid; i <= n; i += 256) s_cu[i] = p.cu_seqlens[i];
    __syncthreads();
    auto cu = [&](int i) { return cached ? s_cu[i] : p.cu_seqlens[i]; };
    // every thread checks and counts the chunks of a contiguous block of
    // sequences; then the block counts are prefix-summed
    const int per = (n + 255) / 256;
    const int s0 = min(n, tid * per), s1 = min(n, s0 + per);
    long long cnt = 0;
    bool bad = tid == 0 && !(cu(0) == 0 && cu(n) == p.seqlen);
    for (int s = s0; s < s1; ++s) {
        const int a = cu(s), e = cu(s + 1);
        bad = bad || !(a >= 0 && e >= a && e <= p.seqlen);
        cnt += (e > a) ? ((long long)e - a + Q - 1) / Q : 0;
    }
    s_part[tid] = cnt;
    if (bad) atomicOr(&s_bad, 1);
    __syncthreads();
    if (tid == 0) {
        long long acc = 0;
        for (int t = 0; t < 256; ++t) {
            const long long v = s_part[t];
            s_part[t] = acc;
            acc += v;
        }
        const bool ok = !s_bad && acc <= p.max_entries;
        if (!ok) {
            *p.error |= 2;
            acc = 0;
            s_bad = 1;
        }
        p.seq_chunk_start[n] = (int)acc;
        if (cached) s_cs[n] = (int)acc;
        *p.n_chunks = (int)acc;
    }
    __syncthreads();
    if (s_bad) return false;
    {
        long long acc = s_part[tid];
        for (int s = s0; s < s1; ++s) {
            const int a = cu(s), e = cu(s + 1);
            p.seq_chunk_start[s] = (int)acc;
            if (cached) s_cs[s] = (int)acc;
            acc += (e > a) ? ((long long)e - a + Q - 1) / Q : 0;
        }
    }
    __syncthreads();
    auto cs = [&](int i) { return cached ? s_cs[i] : p.seq_chunk_start[i]; };
    const int total = cs(n);
    for (int f = tid; f < total; f += 256) {
        int lo = 0, hi = n - 1;  // last s with seq_chunk_start[s] <= f
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cs(mid) <= f) lo = mid; else hi = mid - 1;
        }
        const int s = lo;
        const int c = f - cs(s);
        // position in chunk-index-major order
        int idx = 0;
        for (int t = 0; t < n; ++t) {
            const int nct = cs(t + 1) - cs(t);
            idx += min(nct, c) + ((t < s && nct > c) ? 1 : 0);
        }
        const int start = cu(s) + c * Q;
        const int len = min(Q, cu(s + 1) - start);
        p.chunks[idx] = make_int4(s, c, start, len | (start + len == cu(s + 1) ? ssd::kLastChunk : 0));
    }
    if (p.final_state) {
        for (int s = 0; s < n; ++s) {
            if (cu(s + 1) > cu(s)) continue;
            const long long base = (long long)s * p.H * p.state_elems;
            for (long long k = tid; k < (long long)p.H * p.state_elems; k += 256)
                p.final_state[base + k] = p.init_state ? p.init_state[base + k] : 0.f;
        }
    }
    return true;
}

__global__ __launch_bounds__(256) void ssd_prep_kernel(PrepParams p) {
    const int tid = threadIdx.x;
    const int Q = p.Q;
    __shared__ int cnt[16], run[16];
    for (int u = tid; u < p.nseq * p.H; u += 256) p.flags[(long long)u * p.flag_stride] = 0;
    if (tid < 16) {
        p.tickets[tid] = 0;
        cnt[tid] = 0;
        run[tid] = 0;
    }
    if (tid == 0) *p.error = 0;
    if (p.cu_seqlens == nullptr) {
        const int nc = (p.seqlen + Q - 1) / Q;
        const int total = nc * p.batch;
        if (tid == 0) *p.n_chunks = total;
        for (int e = tid; e < total; e += 256) {
            const int c = e / p.batch;
            const int s = e - c * p.batch;
            const int start = c * Q;
            const int len = min(Q, p.seqlen - start);
            p.chunks[e] = make_int4(s, c, s * p.seqlen + start, len | (c == nc - 1 ? ssd::kLastChunk : 0));
        }
    } else {
        build_packed_schedule(p);   // an invalid table leaves zero entries
    }
    __syncthreads();
    // per-XCD item lists: counts, offsets, then an order-preserving placement.
    // The sequence of each entry is cached in LDS (the placement loop would
    // otherwise wait on one global load per step).
    constexpr int kSeqCache = 4096;
    __shared__ int sseq[kSeqCache];
    const int n_entries = *p.n_chunks;
    const bool dense = p.cu_seqlens == nullptr;
    for (int e = tid; e < n_entries && e < kSeqCache; e += 256) sseq[e] = dense ? e % p.batch : p.chunks[e].x;
    __syncthreads();
    const int GS = p.G * p.slices;
    const int n_items = n_entries * GS;
    const int n_chains = p.nseq * GS;
    if (dense && n_chains % p.n_xcd == 0) {
        // XCD x runs chains [x per, (x + 1) per) of the (sequence, group,
        // slice) order; for every chunk index it holds one item per chain, in
        // chain order, which is also the entry order (closed form)
        const int per = n_chains / p.n_xcd;
        const int nc = n_entries / p.nseq;
        if (tid < 16) {
            p.xcd_count[tid] = tid < p.n_xcd ? nc * per : 0;
            p.xcd_offset[tid] = (tid < p.n_xcd ? tid : p.n_xcd) * nc * per;
        }
        for (int i = tid; i < n_items; i += 256) {
            const int e = i / GS;
            const int j = i - e * GS;
            const int c = e / p.nseq;
            const int k = (e - c * p.nseq) * GS + j;   // chain
            const int x = k / per;
            p.items[x * nc * per + c * per + (k - x * per)] = i;
        }
        return;
    }
    if (!dense && GS % p.n_xcd == 0) {
        // item j of every entry goes to XCD j mod n_xcd (the sequence term is
        // a multiple of n_xcd): the lists have a closed form, written in parallel
        const int per = GS / p.n_xcd;
        if (tid < 16) {
            p.xcd_count[tid] = tid < p.n_xcd ? n_entries * per : 0;
            p.xcd_offset[tid] = (tid < p.n_xcd ? tid : p.n_xcd) * n_entries * per;
        }
        for (int i = tid; i < n_items; i += 256) {
            const int e = i / GS;
            const int j = i - e * GS;
            const int x = j % p.n_xcd;
            p.items[x * n_entries * per + e * per + j / p.n_xcd] = i;
        }
        return;
    }
    auto xcd_of = [&](int i) {
        const int e = i / GS;
        const int seq = e < kSeqCache ? sseq[e] : p.chunks[e].x;
        const long long k = (long long)seq * GS + (i - e * GS);   // chain
        return dense ? (int)(k * p.n_xcd / n_chains) : (int)(k % p.n_xcd);
    };
    for (int i = tid; i < n_items; i += 256) atomicAdd(&cnt[xcd_of(i)], 1);
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int x = 0; x < 16; ++x) {
            p.xcd_offset[x] = acc;
            p.xcd_count[x] = cnt[x];
            acc += cnt[x];
            cnt[x] = p.xcd_offset[x];
        }
    }
    __syncthreads();
    if (tid < 64) {
        const unsigned long long lt = (1ull << tid) - 1ull;
        for (int base = 0; base < n_items; base += 64) {
            const int i = base + tid;
            const bool valid = i < n_items;
            const int x = valid ? xcd_of(i) : 0;
            unsigned long long same = __ballot(valid);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const unsigned long long m = __ballot(valid && ((x >> b) & 1));
                same &= ((x >> b) & 1) ? m : ~m;
            }
            const int rank = __popcll(same & lt);
            volatile int *vrun = run;
            if (valid) p.items[cnt[x] + vrun[x] + rank] = i;
            __builtin_amdgcn_wave_barrier();
            if (valid && rank == 0) vrun[x] = vrun[x] + __popcll(same);
            __builtin_amdgcn_wave_barrier();
        }
    }
}

// ---------------------------------------------------------------------------
// Decode: one workgroup per (batch row, head).  Each thread owns four
// consecutive state columns (one 16-byte vector) of several state rows; the
// P x N fp32 state is streamed once (read, updated, written back in place by
// the same lane, so there is no read-after-write hazard), and the per-row
// read-out C . h is reduced across the N/4 lanes that share the row.
struct DecodeParams {
    float *state;
    const void *x;
    const float *dt;
    DtProc dtp;
    const float *A;
    const void *B;
    const void *C;
    const float *D;
    void *y;
    int H, G, P;
};

template <typename IO, int N>
__global__ __launch_bounds__(256) void ssd_decode_kernel(DecodeParams p) {
    constexpr int C4 = N / 4;          // lanes per state row
    constexpr int RPP = 256 / C4;      // rows per pass of the workgroup
    constexpr int UNR = (64 / RPP) > 0 ? (64 / RPP) : 1;  // passes kept in flight
    const int u = blockIdx.x;
    const int b = u / p.H;
    const int h = u - b * p.H;
    const int g = h / (p.H / p.G);
    const int tid = threadIdx.x;
    const int c4 = tid % C4;
    const int r0 = tid / C4;
    const IO *Bp = reinterpret_cast<const IO *>(p.B) + ((long long)b * p.G + g) * N + 4 * c4;
    const IO *Cp = reinterpret_cast<const IO *>(p.C) + ((long long)b * p.G + g) * N + 4 * c4;
    float bv[4], cv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) { bv[k] = to_f32(Bp[k]); cv[k] = to_f32(Cp[k]); }
    const float d = p.dtp.on ? p.dtp.apply(p.dt[u], p.dtp.bias ? p.dtp.bias[h] : 0.f) : p.dt[u];
    const float abar = __expf(d * p.A[h]);
    const float Dh = p.D ? p.D[h] : 0.f;
    const IO *xp = reinterpret_cast<const IO *>(p.x) + (long long)u * p.P;
    IO *yp = reinterpret_cast<IO *>(p.y) + (long long)u * p.P;
    f32x4 *st = reinterpret_cast<f32x4 *>(p.state + (long long)u * p.P * N);
    for (int base = 0; base < p.P; base += RPP * UNR) {
        f32x4 hv[UNR];
        float xv[UNR];
#pragma unroll
        for (int k = 0; k < UNR; ++k) {
            const int row = base + k * RPP + r0;
            if (row < p.P) {
                hv[k] = __builtin_nontemporal_load(st + (long long)row * C4 + c4);
                xv[k] = to_f32(xp[row]);
            }
        }
#pragma unroll
        for (int k = 0; k < UNR; ++k) {
            const int row = base + k * RPP + r0;
            float part = 0.f;
            if (row < p.P) {
                const float dx = d * xv[k];
                f32x4 nv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    nv[e] = abar * hv[k][e] + dx * bv[e];
                    part += nv[e] * cv[e];
                }
                __builtin_nontemporal_store(nv, st + (long long)row * C4 + c4);
            }
#pragma unroll
            for (int off = C4 / 2; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
            if (row < p.P && c4 == 0) yp[row] = from_f32<IO>(part + Dh * xv[k]);
        }
    }
}

template <typename IO>
static bool decode_launch(int N, const DecodeParams &prm, unsigned grid, hipStream_t st) {
    switch (N) {
    case 16: hipLaunchKernelGGL((ssd_decode_kernel<IO, 16>), dim3(grid), dim3(256), 0, st, prm); return true;
    case 32: hipLaunchKernelGGL((ssd_decode_kernel<IO, 32>), dim3(grid), dim3(256), 0, st, prm); return true;
    case 64: hipLaunchKernelGGL((ssd_decode_kernel<IO, 64>), dim3(grid), dim3(256), 0, st, prm); return true;
    case 128: hipLaunchKernelGGL((ssd_decode_kernel<IO, 128>), dim3(grid), dim3(256), 0, st, prm); return true;
    case 256: hipLaunchKernelGGL((ssd_decode_kernel<IO, 256>), dim3(grid), dim3(256), 0, st, prm); return true;
    default: return false;
    }
}

template <typename IO>
static bool conv_launch(int width, const ConvParams &p, dim3 grid, hipStream_t st) {
    switch (width) {
    case 1: hipLaunchKernelGGL((ssd_conv1d_kernel<IO, 1>), grid, dim3(256), 0, st, p); return true;
    case 2: hipLaunchKernelGGL((ssd_conv1d_kernel<IO, 2>), grid, dim3(256), 0, st, p); return true;
    case 3: hipLaunchKernelGGL((ssd_conv1d_kernel<IO, 3>), grid, dim3(256), 0, st, p); return true;
    case 4: hipLaunchKernelGGL((ssd_conv1d_kernel<IO, 4>), grid, dim3(256), 0, st, p); return true;
    default: return false;
    }
}

// Backward: kernel head dims 16..64 with dstate 16..128 (bf16) or 16..64
// (fp32), where the chunk kernel's tiles fit in LDS (head dim 128 runs as two
// kernel heads of 64).
template <typename IO, int P, int N>
static bool bwd_try(int pp, int nn, const BwdParams &p, unsigned units, unsigned n_chunks_max, bool launch,
                    hipStream_t st) {
    if (pp != P || nn != N) return false;
    if (launch) {
        if constexpr (sizeof(IO) == 2 && P >= 32 && N >= 32) {
            hipLaunchKernelGGL((ssd_bwd_scan_bf16_kernel<P, N>), dim3(2 * units), dim3(256), 0, st, p);
        } else {
            hipLaunchKernelGGL((ssd_bwd_scan_kernel<IO, P, N, 0>), dim3(units), dim3(256), 0, st, p);
            hipLaunchKernelGGL((ssd_bwd_scan_kernel<IO, P, N, 1>), dim3(units), dim3(256), 0, st, p);
        }
        if constexpr (sizeof(IO) == 2 && P >= 32 && N >= 32)
            hipLaunchKernelGGL((ssd_bwd_chunk_bf16_kernel<P, N, kBwdChunkWaves>), dim3(n_chunks_max * (unsigned)p.G),
                               dim3(64 * kBwdChunkWaves), 0, st, p);
        else
            hipLaunchKernelGGL((ssd_bwd_chunk_kernel<IO, P, N>), dim3(n_chunks_max * (unsigned)p.G), dim3(256), 0,
                               st, p);
    }
    return true;
}

template <typename IO, int P>
static bool bwd_try_n(int pp, int nn, const BwdParams &p, unsigned units, unsigned ncm, bool launch,
                      hipStream_t st) {
    if constexpr (sizeof(IO) == 2) {
        return bwd_try<IO, P, 16>(pp, nn, p, units, ncm, launch, st) ||
               bwd_try<IO, P, 32>(pp, nn, p, units, ncm, launch, st) ||
               bwd_try<IO, P, 64>(pp, nn, p, units, ncm, launch, st) ||
               bwd_try<IO, P, 128>(pp, nn, p, units, ncm, launch, st);
    } else {
        return bwd_try<IO, P, 16>(pp, nn, p, units, ncm, launch, st) ||
               bwd_try<IO, P, 32>(pp, nn, p, units, ncm, launch, st) ||
               bwd_try<IO, P, 64>(pp, nn, p, units, ncm, launch, st);
    }
}

template <typename IO>
static bool bwd_dispatch(int pp, int nn, const BwdParams &p, unsigned units, unsigned ncm, bool launch,
                         hipStream_t st) {
    return bwd_try_n<IO, 16>(pp, nn, p, units, ncm, launch, st) ||
           bwd_try_n<IO, 32>(pp, nn, p, units, ncm, launch, st) ||
           bwd_try_n<IO, 64>(pp, nn, p, units, ncm, launch, st);
}

template <typename IO, int NCH>
static bool norm_try(int nch, int mode, const NormParams &p, unsigned blocks, hipStream_t st) {
    if (nch != NCH) return false;
    switch (mode) {
    case 0: hipLaunchKernelGGL((ssd_gated_norm_kernel<IO, NCH, 0>), dim3(blocks), dim3(256), 0, st, p); break;
    case 1: hipLaunchKernelGGL((ssd_gated_norm_kernel<IO, NCH, 1>), dim3(blocks), dim3(256), 0, st, p); break;
    default: hipLaunchKernelGGL((ssd_gated_norm_kernel<IO, NCH, 2>), dim3(blocks), dim3(256), 0, st, p); break;
    }
    return true;
}

template <typename IO, int... NCH>
static bool norm_dispatch(int nch, int mode, const NormParams &p, unsigned blocks, hipStream_t st,
                          std::integer_sequence<int, NCH...>) {
    return (norm_try<IO, NCH + 1>(nch, mode, p, blocks, st) || ...);
}

// one wave per (row, group), 512 channels per register chunk: 1..16 chunks
// for bf16 io, 1..8 for fp32; mode 0 no gate, 1 gate before the norm, 2 after
template <typename IO>
static bool norm_launch(int nch, int mode, const NormParams &p, unsigned blocks, hipStream_t st) {
    return norm_dispatch<IO>(nch, mode, p, blocks, st, std::make_integer_sequence<int, sizeof(IO) == 2 ? 16 : 8>{});
}

}  // namespace ssd

// ===========================================================================
// C ABI
namespace {

// Scratch of ssd_chunk_scan_fwd_noalloc: the workspace of one call (header,
// progress flags, chunk table, item lists and, when the caller passes no
// final_state, the boundary states), in a file-scope device array so that
// the call allocates nothing.  Each device holds its own copy for the life
// of the process; host code reaches it only through the address that
// hipGetSymbolAddress returns for the current device (the array's name is a
// host-side stand-in, not a device address).
constexpr size_t kNoAllocScratchBytes = SSD_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

// This device's address of `scratch`, looked up on the first call on each
// device (with that device current) and cached; SSD_ERR_HIP if the runtime
// cannot resolve it.  Concurrent first calls store the same address.
ssd_status_t scratch_base(char **out) {
    static std::atomic<char *> cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SSD_ERR_HIP;
    const bool cached = dev >= 0 && dev < 64;
    if (cached) {
        char *c = cache[dev].load(std::memory_order_acquire);
        if (c) {
            *out = c;
            return SSD_OK;
        }
    }
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return SSD_ERR_HIP;
    if (cached) cache[dev].store(static_cast<char *>(ptr), std::memory_order_release);
    *out = static_cast<char *>(ptr);
    return SSD_OK;
}

struct Range {
    uintptr_t lo, hi;
};

Range rng(const void *p, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + bytes};
}

bool overlap(Range a, Range b) {
    if (a.lo == 0 || b.lo == 0 || a.hi == a.lo || b.hi == b.lo) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

// A device attribute of the current device (cached per device id), or -1.
// The cache only ever holds the attribute's value, so concurrent first calls
// store the same number; the accesses are atomic to keep that race defined.
int device_attr(hipDeviceAttribute_t attr, std::atomic<int> (&cache)[64]) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (dev >= 0 && dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, attr, dev) != hipSuccess || n <= 0) return -1;
    if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

int num_compute_units() {
    static std::atomic<int> cache[64] = {};
    return device_attr(hipDeviceAttributeMultiprocessorCount, cache);
}

// Number of XCDs (accelerator complexes, each with its own L2) of the
// current device, clamped to at most 16, or -1 when the runtime cannot tell.
// The forward's hand-off keeps every chain on one XCD, so a wrong count is an
// error, never silently replaced by a default.
int num_xcds() {
    static std::atomic<int> cache[64] = {};
    const int n = device_attr(hipDeviceAttributeNumberOfXccs, cache);
    return n < 1 ? -1 : (n > 16 ? 16 : n);
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Optional check of the packed-sequence offsets, enabled by the environment
// variable SSD_DEBUG_VALIDATE=1: copies them to the host (which synchronises
// `s`) and requires cu[0] == 0, non-decreasing entries and cu[nseq] ==
// seqlen.  Without the variable these are unchecked preconditions.
ssd_status_t debug_check_cu_seqlens(const int32_t *cu, int nseq, int seqlen, hipStream_t s) {
    const char *flag = std::getenv("SSD_DEBUG_VALIDATE");
    if (!cu || !flag || std::strcmp(flag, "1") != 0) return SSD_OK;
    std::vector<int32_t> h((size_t)nseq + 1);
    if (hipMemcpyAsync(h.data(), cu, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess)
        return SSD_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return SSD_ERR_HIP;
    if (h[0] != 0 || h[(size_t)nseq] != seqlen) return SSD_ERR_SHAPE;
    for (int i = 0; i < nseq; ++i)
        if (h[(size_t)i + 1] < h[(size_t)i]) return SSD_ERR_SHAPE;
    return SSD_OK;
}

// The forward kernel's view of the heads: head dim 128 runs as two kernel
// heads of 64 channels each (x, y and the states then have exactly the layout
// of twice the heads at half the head dim; the kernel indexes dt, A, D and
// dt_bias by the model head).
struct KHeads {
    int H, P, hsub;
};

KHeads kernel_heads(const ssd_dims_t &d) {
    const int hsub = d.headdim == 128 ? 2 : 1;
    return KHeads{d.nheads * hsub, d.headdim / hsub, hsub};
}

struct WsLayout {
    size_t flags, chunks, items, scratch, state, total;
    long long max_entries;
};

// Workspace header (bytes): [0,64) one ticket per XCD, 64 error word,
// 68 entry count, [128,192) items per XCD, [192,256) list offsets.
constexpr size_t kWsTickets = 0, kWsError = 64, kWsEntries = 68, kWsXcdCount = 128, kWsXcdOffset = 192;

// Progress flags one 128-byte line apart while they take at most 4 MiB: the
// workgroups of an XCD poll and bump the flags of neighbouring heads at the
// same time, and flags sharing a line serialize those accesses (130M-layer
// shape 96 -> 87 us).  Beyond that, packed.
int flag_stride(const ssd_dims_t &d) {
    return (long long)d.nseq * kernel_heads(d).H <= 32768 ? 32 : 1;
}

// Workspace: header; per-(sequence, head) flags; chunk table; per-XCD item
// lists (at most entries x heads items); packed-batch scratch; fp32
// boundary-state buffer.
bool ws_layout(const ssd_dims_t &d, int Q, bool varlen, WsLayout *w) {
    const long long nc = ((long long)d.seqlen + Q - 1) / Q;
    const int kh = kernel_heads(d).H;
    w->max_entries = varlen ? nc + d.nseq : nc * d.batch;
    w->flags = 256;
    w->chunks = align_up(w->flags + (size_t)d.nseq * kh * 4 * flag_stride(d), 256);
    w->items = align_up(w->chunks + (size_t)w->max_entries * 16, 256);
    w->scratch = align_up(w->items + (size_t)w->max_entries * kh * 4, 256);
    w->state = align_up(w->scratch + (size_t)(d.nseq + 1) * 4, 256);
    w->total = align_up(w->state + (size_t)d.nseq * d.nheads * d.headdim * d.dstate * 4, 256);
    return true;
}

bool dims_ok(const ssd_dims_t &d) {
    return d.batch >= 1 && d.seqlen >= 1 && d.nheads >= 1 && d.headdim >= 1 && d.dstate >= 1 &&
           d.ngroups >= 1 && d.nseq >= 1 && d.nheads % d.ngroups == 0;
}

// Validates the step-size options and fills the kernels' view of them.
ssd_status_t dt_opts_check(const ssd_dt_opts_t *o, const ssd_dims_t &d, ssd::DtProc *out) {
    (void)d;
    *out = ssd::DtProc{};
    if (!o) return SSD_OK;
    if (!(o->dt_min <= o->dt_max)) return SSD_ERR_SHAPE;   // also rejects NaN bounds
    out->bias = o->dt_bias;
    out->softplus = o->softplus != 0;
    out->lo = o->dt_min;
    out->hi = o->dt_max;
    out->on = o->dt_bias != nullptr || o->softplus != 0 || o->dt_min > -INFINITY || o->dt_max < INFINITY;
    return SSD_OK;
}

// The chunk length the kernel runs for a requested chunk_len: chunk_len
// itself where its tiles fit in LDS, else the largest smaller one (at least
// 64) that fits, or 0 when none is built.  Chunking only orders the
// evaluation (the result is the recurrence's either way, up to rounding).
int kernel_chunk(const ssd_dims_t &d, int32_t chunk_len, ssd_dtype_t io) {
    ssd::FwdParams dummy{};
    hipError_t e = hipSuccess;
    for (int q = chunk_len; q >= 64; q /= 2) {
        const bool built = (io == SSD_BF16)
                               ? ssd::fwd_dispatch_bf16(kernel_heads(d).P, d.dstate, q, dummy, 0, nullptr, false, &e)
                               : ssd::fwd_dispatch_f32(kernel_heads(d).P, d.dstate, q, dummy, 0, nullptr, false, &e);
        if (built) return q;
    }
    return 0;
}

ssd_status_t fwd_shape_check(const ssd_dims_t *dims, int32_t chunk_len, ssd_dtype_t io, bool varlen) {
    if (!dims) return SSD_ERR_NULL_PTR;
    if (io != SSD_F32 && io != SSD_BF16) return SSD_ERR_DTYPE;
    const ssd_dims_t &d = *dims;
    if (!dims_ok(d)) return SSD_ERR_SHAPE;
    if (varlen) {
        if (d.batch != 1 || d.nseq > 65536) return SSD_ERR_SHAPE;
    } else if (d.nseq != d.batch) {
        return SSD_ERR_SHAPE;
    }
    if (chunk_len != 64 && chunk_len != 128 && chunk_len != 256) return SSD_ERR_UNSUPPORTED;
    if (kernel_chunk(d, chunk_len, io) == 0) return SSD_ERR_UNSUPPORTED;
    // sizes must stay within the kernels' 32-bit schedule fields
    const long long tokens = (long long)d.batch * d.seqlen;
    if (tokens > INT_MAX / 2) return SSD_ERR_SHAPE;
    // one chunk of x (or y) rows, all heads, must span less than 2^30 bytes:
    // the kernel addresses it through a buffer with 30-bit offsets
    if ((long long)d.nheads * d.headdim * 256 * 4 >= (1LL << 30)) return SSD_ERR_SHAPE;
    return SSD_OK;
}

}  // namespace

extern "C" {

const char *ssd_status_string(ssd_status_t s) {
    switch (s) {
    case SSD_OK: return "SSD_OK";
    case SSD_ERR_NULL_PTR: return "SSD_ERR_NULL_PTR: a required pointer is NULL";
    case SSD_ERR_SHAPE: return "SSD_ERR_SHAPE: invalid or inconsistent dimensions";
    case SSD_ERR_DTYPE: return "SSD_ERR_DTYPE: unknown io dtype";
    case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED: headdim/dstate/chunk_len combination not built";
    case SSD_ERR_ALIGNMENT: return "SSD_ERR_ALIGNMENT: pointer not sufficiently aligned";
    case SSD_ERR_ALIAS: return "SSD_ERR_ALIAS: an output overlaps an input";
    case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE: workspace missing or too small";
    case SSD_ERR_HIP: return "SSD_ERR_HIP: HIP runtime error";
    case SSD_ERR_DEVICE: return "SSD_ERR_DEVICE: a kernel reported an internal failure";
    }
    return "SSD status: unknown code";
}

int32_t ssd_abi_version(void) { return SSD_ABI_VERSION; }

size_t ssd_chunk_scan_fwd_workspace_size(const ssd_dims_t *dims, int32_t chunk_len, ssd_dtype_t io) {
    if (!dims) return 0;
    // the size query does not know whether cu_seqlens will be passed: accept
    // either reading of the dims and size for the larger (packed) schedule
    if (fwd_shape_check(dims, chunk_len, io, true) != SSD_OK &&
        fwd_shape_check(dims, chunk_len, io, false) != SSD_OK)
        return 0;
    WsLayout packed{}, dense{};
    const int q = kernel_chunk(*dims, chunk_len, io);
    ws_layout(*dims, q, true, &packed);
    ws_layout(*dims, q, false, &dense);
    return packed.total > dense.total ? packed.total : dense.total;
}

ssd_status_t ssd_chunk_scan_fwd(const ssd_dims_t *dims, ssd_dtype_t io, int32_t chunk_len,
                                const void *x, const float *dt, const float *A, const void *B,
                                const void *C, const float *D, const float *init_state,
                                const int32_t *cu_seqlens, void *y, float *final_state,
                                void *workspace, size_t workspace_bytes, void *stream) {
    return ssd_chunk_scan_fwd_ex(dims, io, chunk_len, nullptr, x, dt, A, B, C, D, init_state, cu_seqlens, y,
                                 final_state, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {
// The forward entry points.  `scratch_mode` runs the call on this device's
// copy of the file-scope scratch array instead of a caller workspace
// (`workspace` and `workspace_bytes` are then ignored).
ssd_status_t fwd_impl(const ssd_dims_t *dims, ssd_dtype_t io, int32_t chunk_len, const ssd_dt_opts_t *dt_opts,
                      const void *x, const float *dt, const float *A, const void *B, const void *C,
                      const float *D, const float *init_state, const int32_t *cu_seqlens, void *y,
                      float *final_state, void *workspace, size_t workspace_bytes, bool scratch_mode,
                      void *stream) {
    const bool varlen = cu_seqlens != nullptr;
    ssd_status_t st = fwd_shape_check(dims, chunk_len, io, varlen);
    if (st != SSD_OK) return st;
    chunk_len = kernel_chunk(*dims, chunk_len, io);
    ssd::DtProc dtp{};
    st = dt_opts_check(dt_opts, *dims, &dtp);
    if (st != SSD_OK) return st;
    const ssd_dims_t &d = *dims;
    if (!x || !dt || !A || !B || !C || !y) return SSD_ERR_NULL_PTR;
    if (!scratch_mode && !workspace) return SSD_ERR_WORKSPACE;
    const void *al16[] = {x, dt, A, B, C, D, init_state, y, final_state, dtp.bias};
    for (const void *p : al16)
        if (p && !aligned(p, 16)) return SSD_ERR_ALIGNMENT;
    if (!scratch_mode && !aligned(workspace, 256)) return SSD_ERR_ALIGNMENT;
    if (cu_seqlens && !aligned(cu_seqlens, 4)) return SSD_ERR_ALIGNMENT;

    const size_t E = (io == SSD_BF16) ? 2 : 4;
    const size_t tokens = (size_t)d.batch * d.seqlen;
    const size_t nx = tokens * d.nheads * d.headdim * E;
    const size_t nbc = tokens * d.ngroups * d.dstate * E;
    const size_t nstate = (size_t)d.nseq * d.nheads * d.headdim * d.dstate * 4;
    const Range ry = rng(y, nx);
    const Range rx = rng(x, nx), rdt = rng(dt, tokens * d.nheads * 4), rA = rng(A, (size_t)d.nheads * 4);
    const Range rB = rng(B, nbc), rC = rng(C, nbc), rD = rng(D, D ? (size_t)d.nheads * 4 : 0);
    const Range ri = rng(init_state, init_state ? nstate : 0), rf = rng(final_state, final_state ? nstate : 0);
    const Range rcu = rng(cu_seqlens, cu_seqlens ? (size_t)(d.nseq + 1) * 4 : 0);
    const Range rbias = rng(dtp.bias, dtp.bias ? (size_t)d.nheads * 4 : 0);
    if (overlap(ry, rbias) || overlap(rf, rbias)) return SSD_ERR_ALIAS;
    WsLayout w{};
    ws_layout(d, chunk_len, varlen, &w);
    if (scratch_mode) {
        // the boundary-state part is needed only when final_state is NULL
        if ((final_state ? w.state : w.total) > kNoAllocScratchBytes) return SSD_ERR_WORKSPACE;
    } else if (workspace_bytes < w.total) {
        return SSD_ERR_WORKSPACE;
    }
    // (the scratch array is the library's own memory: no caller buffer can
    // overlap it, so these checks pass in scratch mode)
    const Range rw = rng(workspace, scratch_mode ? 0 : w.total);
    for (Range r : {rx, rdt, rA, rB, rC, rD, ri, rf, rcu, rw})
        if (overlap(ry, r)) return SSD_ERR_ALIAS;
    for (Range r : {rx, rdt, rA, rB, rC, rD, rcu, rw})
        if (overlap(rf, r)) return SSD_ERR_ALIAS;   // final_state may equal init_state
    if (final_state && init_state && overlap(rf, ri) && rf.lo != ri.lo) return SSD_ERR_ALIAS;
    for (Range r : {rx, rdt, rA, rB, rC, rD, ri, rcu})
        if (overlap(rw, r)) return SSD_ERR_ALIAS;
    const KHeads kh = kernel_heads(d);
    if (w.max_entries * kh.H > INT_MAX || (long long)d.nseq * kh.H > INT_MAX) return SSD_ERR_SHAPE;
    if (scratch_mode) {
        char *base = nullptr;
        const ssd_status_t sst = scratch_base(&base);
        if (sst != SSD_OK) return sst;
        workspace = base;
    }

    char *ws = static_cast<char *>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = debug_check_cu_seqlens(cu_seqlens, d.nseq, d.seqlen, s);
    if (st != SSD_OK) return st;
    ssd::PrepParams pp{};
    pp.cu_seqlens = cu_seqlens;
    pp.batch = d.batch;
    pp.seqlen = d.seqlen;
    pp.nseq = d.nseq;
    pp.H = kh.H;
    pp.Q = chunk_len;
    pp.state_elems = kh.P * d.dstate;
    pp.chunks = reinterpret_cast<int4 *>(ws + w.chunks);
    pp.n_chunks = reinterpret_cast<int *>(ws + kWsEntries);
    pp.tickets = reinterpret_cast<int *>(ws + kWsTickets);
    pp.error = reinterpret_cast<int *>(ws + kWsError);
    pp.flags = reinterpret_cast<int *>(ws + w.flags);
    pp.items = reinterpret_cast<int *>(ws + w.items);
    pp.xcd_count = reinterpret_cast<int *>(ws + kWsXcdCount);
    pp.xcd_offset = reinterpret_cast<int *>(ws + kWsXcdOffset);
    pp.seq_chunk_start = reinterpret_cast<int *>(ws + w.scratch);
    pp.init_state = init_state;
    pp.final_state = final_state;

    // head slice per work item: about eight items per compute unit, so that
    // the workgroups sharing an XCD walk many different heads at a time
    const int cus = num_compute_units();
    if (cus <= 0) return SSD_ERR_HIP;
    const int hpg = kh.H / d.ngroups;
    const long long want = 8LL * cus;
    long long hs = (w.max_entries * kh.H + want - 1) / want;
    hs = hs < 1 ? 1 : (hs > hpg ? hpg : hs);
    // but at least three heads where the group has them: an item's set-up
    // (its B and C rows, the C B^T tiles) costs more than one head (at the
    // 130M-layer shape 3-head items ran 97 us, 2-head 101, 6-head 122)
    if (hs < 3) hs = hpg < 3 ? hpg : 3;
    const int slices = (int)((hpg + hs - 1) / hs);
    pp.G = d.ngroups;
    pp.slices = slices;
    pp.max_entries = (int)w.max_entries;
    pp.n_xcd = num_xcds();
    if (pp.n_xcd < 1) return SSD_ERR_HIP;
    pp.flag_stride = flag_stride(d);
    hipLaunchKernelGGL(ssd::ssd_prep_kernel, dim3(1), dim3(256), 0, s, pp);
    if (hipGetLastError() != hipSuccess) return SSD_ERR_HIP;

    ssd::FwdParams fp{};
    fp.x = x;
    fp.dt = dt;
    fp.dtp = dtp;
    fp.A = A;
    fp.B = B;
    fp.C = C;
    fp.D = D;
    fp.init_state = init_state;
    fp.y = y;
    fp.state = final_state ? final_state : reinterpret_cast<float *>(ws + w.state);
    fp.chunks = pp.chunks;
    fp.n_chunks = pp.n_chunks;
    fp.tickets = pp.tickets;
    fp.items = pp.items;
    fp.xcd_count = pp.xcd_count;
    fp.xcd_offset = pp.xcd_offset;
    fp.n_xcd = pp.n_xcd;
    fp.flags = pp.flags;
    fp.flag_stride = pp.flag_stride;
    fp.error = pp.error;
    fp.H = kh.H;
    fp.hsub = kh.hsub;
    fp.G = d.ngroups;
    fp.heads_per_item = (int)hs;
    fp.slices = slices;
    hipError_t err = hipSuccess;
    const bool ok = (io == SSD_BF16)
                        ? ssd::fwd_dispatch_bf16(kh.P, d.dstate, chunk_len, fp, w.max_entries, s, true, &err)
                        : ssd::fwd_dispatch_f32(kh.P, d.dstate, chunk_len, fp, w.max_entries, s, true, &err);
    if (!ok) return SSD_ERR_UNSUPPORTED;
    if (err != hipSuccess) return SSD_ERR_HIP;
    return SSD_OK;
}
}  // namespace

extern "C" {

ssd_status_t ssd_chunk_scan_fwd_ex(const ssd_dims_t *dims, ssd_dtype_t io, int32_t chunk_len,
                                   const ssd_dt_opts_t *dt_opts, const void *x, const float *dt,
                                   const float *A, const void *B, const void *C, const float *D,
                                   const float *init_state, const int32_t *cu_seqlens, void *y,
                                   float *final_state, void *workspace, size_t workspace_bytes,
                                   void *stream) {
    return fwd_impl(dims, io, chunk_len, dt_opts, x, dt, A, B, C, D, init_state, cu_seqlens, y, final_state,
                    workspace, workspace_bytes, false, stream);
}

ssd_status_t ssd_chunk_scan_fwd_noalloc(const ssd_dims_t *dims, ssd_dtype_t io, int32_t chunk_len,
                                        const ssd_dt_opts_t *dt_opts, const void *x, const float *dt,
                                        const float *A, const void *B, const void *C, const float *D,
                                        const float *init_state, const int32_t *cu_seqlens, void *y,
                                        float *final_state, void *stream) {
    return fwd_impl(dims, io, chunk_len, dt_opts, x, dt, A, B, C, D, init_state, cu_seqlens, y, final_state,
                    nullptr, 0, true, stream);
}

ssd_status_t ssd_chunk_scan_fwd_check(const void *workspace, void *stream) {
    if (!workspace) return SSD_ERR_WORKSPACE;
    int32_t hdr[64] = {};   // the 256-byte workspace header
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipStreamSynchronize(s) != hipSuccess) return SSD_ERR_HIP;
    if (hipMemcpy(hdr, workspace, sizeof(hdr), hipMemcpyDeviceToHost) != hipSuccess) return SSD_ERR_HIP;
    const int32_t word = hdr[kWsError / 4];
    if (word & 2) return SSD_ERR_SHAPE;
    if (word) return SSD_ERR_DEVICE;
    // every XCD's item list must have been drained: a workgroup takes tickets
    // until one lies past its list, so the counter ends at or beyond the count
    // exactly when every item of the list was taken (and so completed)
    for (int x = 0; x < 16; ++x)
        if (hdr[(kWsTickets / 4) + x] < hdr[(kWsXcdCount / 4) + x]) return SSD_ERR_DEVICE;
    return SSD_OK;
}

ssd_status_t ssd_decode_step(const ssd_dims_t *dims, ssd_dtype_t io, float *state, const void *x,
                             const float *dt, const float *A, const void *B, const void *C,
                             const float *D, void *y, void *stream) {
    return ssd_decode_step_ex(dims, io, nullptr, state, x, dt, A, B, C, D, y, stream);
}

ssd_status_t ssd_decode_step_ex(const ssd_dims_t *dims, ssd_dtype_t io, const ssd_dt_opts_t *dt_opts,
                                float *state, const void *x, const float *dt, const float *A,
                                const void *B, const void *C, const float *D, void *y, void *stream) {
    if (!dims) return SSD_ERR_NULL_PTR;
    if (io != SSD_F32 && io != SSD_BF16) return SSD_ERR_DTYPE;
    const ssd_dims_t &d = *dims;
    if (d.batch < 1 || d.nheads < 1 || d.headdim < 1 || d.dstate < 1 || d.ngroups < 1 ||
        d.nheads % d.ngroups != 0)
        return SSD_ERR_SHAPE;
    ssd::DtProc dtp{};
    ssd_status_t st = dt_opts_check(dt_opts, d, &dtp);
    if (st != SSD_OK) return st;
    const int N = d.dstate;
    if (N != 16 && N != 32 && N != 64 && N != 128 && N != 256) return SSD_ERR_UNSUPPORTED;
    if (!state || !x || !dt || !A || !B || !C || !y) return SSD_ERR_NULL_PTR;
    const void *al16[] = {state, x, dt, A, B, C, D, y, dtp.bias};
    for (const void *p : al16)
        if (p && !aligned(p, 16)) return SSD_ERR_ALIGNMENT;
    const size_t E = (io == SSD_BF16) ? 2 : 4;
    const size_t units = (size_t)d.batch * d.nheads;
    if (units > (size_t)INT_MAX) return SSD_ERR_SHAPE;
    const Range rs = rng(state, units * d.headdim * N * 4);
    const Range rx = rng(x, units * d.headdim * E), ry = rng(y, units * d.headdim * E);
    const Range rdt = rng(dt, units * 4), rA = rng(A, (size_t)d.nheads * 4);
    const Range rB = rng(B, (size_t)d.batch * d.ngroups * N * E), rC = rng(C, (size_t)d.batch * d.ngroups * N * E);
    const Range rD = rng(D, D ? (size_t)d.nheads * 4 : 0);
    for (Range r : {rs, rx, rdt, rA, rB, rC, rD})
        if (overlap(ry, r)) return SSD_ERR_ALIAS;
    for (Range r : {rx, rdt, rA, rB, rC, rD})
        if (overlap(rs, r)) return SSD_ERR_ALIAS;
    const Range rbias = rng(dtp.bias, dtp.bias ? (size_t)d.nheads * 4 : 0);
    if (overlap(ry, rbias) || overlap(rs, rbias)) return SSD_ERR_ALIAS;
    ssd::DecodeParams p{};
    p.state = state;
    p.x = x;
    p.dt = dt;
    p.dtp = dtp;
    p.A = A;
    p.B = B;
    p.C = C;
    p.D = D;
    p.y = y;
    p.H = d.nheads;
    p.G = d.ngroups;
    p.P = d.headdim;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool ok = (io == SSD_BF16) ? ssd::decode_launch<ssd::bf16>(N, p, (unsigned)units, s)
                                     : ssd::decode_launch<float>(N, p, (unsigned)units, s);
    if (!ok) return SSD_ERR_UNSUPPORTED;
    if (hipGetLastError() != hipSuccess) return SSD_ERR_HIP;
    return SSD_OK;
}


ssd_status_t ssd_causal_conv1d_fwd(const ssd_dims_t *dims, ssd_dtype_t io, int32_t width, const void *xbc,
                                   const float *weight, const float *bias, int32_t silu, const void *conv_state,
                                   const int32_t *cu_seqlens, void *x, void *B, void *C, void *conv_state_out,
                                   void *stream) {
    if (!dims) return SSD_ERR_NULL_PTR;
    if (io != SSD_F32 && io != SSD_BF16) return SSD_ERR_DTYPE;
    const ssd_dims_t &d = *dims;
    if (!dims_ok(d)) return SSD_ERR_SHAPE;
    const bool varlen = cu_seqlens != nullptr;
    if (varlen ? d.batch != 1 : d.nseq != d.batch) return SSD_ERR_SHAPE;
    if (width < 1 || width > 4 || d.headdim % 8 != 0 || d.dstate % 8 != 0) return SSD_ERR_UNSUPPORTED;
    if (!xbc || !weight || !x || !B || !C) return SSD_ERR_NULL_PTR;
    const void *al16[] = {xbc, weight, bias, conv_state, x, B, C, conv_state_out};
    for (const void *p : al16)
        if (p && !aligned(p, 16)) return SSD_ERR_ALIGNMENT;
    if (cu_seqlens && !aligned(cu_seqlens, 4)) return SSD_ERR_ALIGNMENT;
    const long long tokens = (long long)d.batch * d.seqlen;
    const long long HP = (long long)d.nheads * d.headdim, GN = (long long)d.ngroups * d.dstate;
    const long long Cc = HP + 2 * GN;
    if (Cc > INT_MAX / 8 || tokens > (long long)INT_MAX) return SSD_ERR_SHAPE;
    const size_t E = (io == SSD_BF16) ? 2 : 4;
    const size_t nst = (size_t)d.nseq * (width - 1) * Cc * E;
    const Range rin = rng(xbc, tokens * Cc * E), rw = rng(weight, Cc * width * 4),
                rb = rng(bias, bias ? Cc * 4 : 0), rs = rng(conv_state, conv_state ? nst : 0),
                rcu = rng(cu_seqlens, varlen ? (size_t)(d.nseq + 1) * 4 : 0);
    const Range rx = rng(x, tokens * HP * E), rB = rng(B, tokens * GN * E), rC = rng(C, tokens * GN * E),
                rso = rng(conv_state_out, conv_state_out ? nst : 0);
    for (Range o : {rx, rB, rC, rso}) {
        for (Range i : {rin, rw, rb, rs, rcu})
            if (overlap(o, i)) return SSD_ERR_ALIAS;
    }
    if (overlap(rx, rB) || overlap(rx, rC) || overlap(rB, rC) || overlap(rso, rx) || overlap(rso, rB) ||
        overlap(rso, rC))
        return SSD_ERR_ALIAS;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const ssd_status_t cst = debug_check_cu_seqlens(cu_seqlens, d.nseq, d.seqlen, st);
    if (cst != SSD_OK) return cst;
    ssd::ConvParams p{};
    p.xbc = xbc;
    p.w = weight;
    p.bias = bias;
    p.state_in = conv_state;
    p.cu_seqlens = cu_seqlens;
    p.x = x;
    p.B = B;
    p.C = C;
    p.state_out = conv_state_out;
    p.tokens = tokens;
    p.seqlen = d.seqlen;
    p.nseq = d.nseq;
    p.Cc = (int)Cc;
    p.HP = (int)HP;
    p.GN = (int)GN;
    p.silu = silu != 0;
    // 32 tokens per thread (two batches of 16), more when the grid would
    // exceed its y limit
    long long run = 32;
    while ((tokens + run * 4 - 1) / (run * 4) > 65535) run *= 2;
    p.run = (int)run;
    const dim3 grid((unsigned)((Cc / 8 + 63) / 64), (unsigned)((tokens + run * 4 - 1) / (run * 4)));
    const bool ok = (io == SSD_BF16) ? ssd::conv_launch<ssd::bf16>(width, p, grid, st)
                                     : ssd::conv_launch<float>(width, p, grid, st);
    if (!ok) return SSD_ERR_UNSUPPORTED;
    if (hipGetLastError() != hipSuccess) return SSD_ERR_HIP;
    return SSD_OK;
}

ssd_status_t ssd_gated_rmsnorm_fwd(int64_t rows, int32_t dim, int32_t group_size, ssd_dtype_t io, const void *y,
                                   const void *z, const float *weight, float eps, int32_t norm_before_gate,
                                   void *out, void *stream) {
    if (io != SSD_F32 && io != SSD_BF16) return SSD_ERR_DTYPE;
    if (rows < 1 || dim < 1 || group_size < 1 || dim % group_size != 0) return SSD_ERR_SHAPE;
    if (!(eps >= 0.f) || !std::isfinite(eps)) return SSD_ERR_SHAPE;
    if (group_size % 8 != 0) return SSD_ERR_UNSUPPORTED;
    const int nch = (group_size + 511) / 512;
    if (nch > ((io == SSD_BF16) ? 16 : 8)) return SSD_ERR_UNSUPPORTED;
    if (!y || !weight || !out) return SSD_ERR_NULL_PTR;
    const void *al16[] = {y, z, weight, out};
    for (const void *p : al16)
        if (p && !aligned(p, 16)) return SSD_ERR_ALIGNMENT;
    const long long groups = dim / group_size;
    const long long units = rows * groups;
    if (rows > LLONG_MAX / dim || (units + 3) / 4 > (long long)INT_MAX) return SSD_ERR_SHAPE;
    const size_t E = (io == SSD_BF16) ? 2 : 4;
    const size_t bytes = (size_t)rows * dim * E;
    const Range ry = rng(y, bytes), rz = rng(z, z ? bytes : 0), rw = rng(weight, (size_t)dim * 4), ro = rng(out, bytes);
    // out may be y or z itself (every group is read whole before it is written)
    if (overlap(ro, rw) || (overlap(ro, ry) && out != y) || (overlap(ro, rz) && out != z)) return SSD_ERR_ALIAS;
    ssd::NormParams p{};
    p.y = y;
    p.z = z;
    p.w = weight;
    p.out = out;
    p.units = units;
    p.dim = dim;
    p.gs = group_size;
    p.groups = (int)groups;
    p.eps = eps;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const unsigned blocks = (unsigned)((units + 3) / 4);
    const int mode = z ? (norm_before_gate ? 2 : 1) : 0;
    const bool ok = (io == SSD_BF16) ? ssd::norm_launch<ssd::bf16>(nch, mode, p, blocks, st)
                                     : ssd::norm_launch<float>(nch, mode, p, blocks, st);
    if (!ok) return SSD_ERR_UNSUPPORTED;
    if (hipGetLastError() != hipSuccess) return SSD_ERR_HIP;
    return SSD_OK;
}


// ---------------------------------------------------------------------------
// Backward pass.
namespace {
struct BwdWs {
    size_t chunks, seqstart, states, radj, partA, partD, total;
    long long max_chunks;
};

bool bwd_ws(const ssd_dims_t &d, bool varlen, BwdWs *w) {
    const long long Q = ssd::kBwdQ;
    const long long per = (d.seqlen + Q - 1) / Q;
    w->max_chunks = varlen ? per + d.nseq : per * d.batch;
    const long long st = (long long)d.nheads * d.headdim * d.dstate * 4;
    w->chunks = 0;
    w->seqstart = align_up((size_t)w->max_chunks * 16, 256);
    w->states = align_up(w->seqstart + (size_t)(d.nseq + 1) * 4, 256);
    w->radj = align_up(w->states + (size_t)(w->max_chunks + d.nseq) * st, 256);
    const long long kh = kernel_heads(d).H;   // per-chunk dA, dD partials per kernel head
    w->partA = align_up(w->radj + (size_t)w->max_chunks * st, 256);
    w->partD = align_up(w->partA + (size_t)w->max_chunks * kh * 4, 256);
    w->total = align_up(w->partD + (size_t)w->max_chunks * kh * 4, 256);
    return true;
}

// State dim of the backward kernels: dstate itself where built, else the
// largest built state dim that divides it (0: none).  Above it the backward
// runs once per slice of the state dim: every state column n evolves on its
// own (h[p, n] depends only on B[:, n]), and y, hence every gradient, is a sum
// over n, so each slice's run gives that slice's columns of dB, dC and dinit
// and one term of dx, ddt and dA (dD does not depend on n).
int bwd_kernel_n(const ssd_dims_t &d, ssd_dtype_t io) {
    const KHeads kh = kernel_heads(d);
    ssd::BwdParams dummy{};
    auto built = [&](int n) {
        return (io == SSD_BF16) ? ssd::bwd_dispatch<ssd::bf16>(kh.P, n, dummy, 0, 0, false, nullptr)
                                : ssd::bwd_dispatch<float>(kh.P, n, dummy, 0, 0, false, nullptr);
    };
    if (built(d.dstate)) return d.dstate;
    if (d.dstate != 128 && d.dstate != 256) return 0;   // the forward's other state dims
    for (int n = 128; n >= 16; n /= 2)
        if (n < d.dstate && d.dstate % n == 0 && built(n)) return n;
    return 0;
}

ssd_status_t bwd_shape_check(const ssd_dims_t *dims, ssd_dtype_t io, bool varlen) {
    if (!dims) return SSD_ERR_NULL_PTR;
    if (io != SSD_F32 && io != SSD_BF16) return SSD_ERR_DTYPE;
    const ssd_dims_t &d = *dims;
    if (!dims_ok(d)) return SSD_ERR_SHAPE;
    if (varlen ? (d.batch != 1 || d.nseq > 65536) : d.nseq != d.batch) return SSD_ERR_SHAPE;
    if (bwd_kernel_n(d, io) == 0) return SSD_ERR_UNSUPPORTED;
    if ((long long)d.batch * d.seqlen > INT_MAX / 2 || (long long)d.nseq * kernel_heads(d).H > INT_MAX)
        return SSD_ERR_SHAPE;
    // the scans address one chunk of x, dy, B or C rows (every head or group)
    // with 32-bit byte offsets
    if ((long long)d.nheads * d.headdim * ssd::kBwdQ * 4 >= (1LL << 30) ||
        (long long)d.ngroups * d.dstate * ssd::kBwdQ * 4 >= (1LL << 30))
        return SSD_ERR_SHAPE;
    return SSD_OK;
}

// Workspace of a state-dim-split backward: the kernels' own workspace for one
// slice, then the slice's inputs (B, C, initial state, final-state gradient),
// its dB, dC and dinit, and every slice's dx, ddt, dA and dD terms.
struct BwdSplitWs {
    size_t B, C, init, dfin, dinit, dB, dC, dx, ddt, dA, dD, total;
    int kn, nsplit;
    BwdWs inner;
};

bool bwd_split_ws(const ssd_dims_t &d, ssd_dtype_t io, bool varlen, BwdSplitWs *w) {
    w->kn = bwd_kernel_n(d, io);
    w->nsplit = w->kn ? d.dstate / w->kn : 0;
    ssd_dims_t dk = d;
    dk.dstate = w->kn;
    bwd_ws(dk, varlen, &w->inner);
    const size_t E = (io == SSD_BF16) ? 2 : 4;
    const size_t tokens = (size_t)d.batch * d.seqlen;
    const size_t nbk = tokens * d.ngroups * w->kn, nstk = (size_t)d.nseq * d.nheads * d.headdim * w->kn * 4;
    const size_t nx = tokens * d.nheads * d.headdim;
    w->B = align_up(w->inner.total, 256);
    w->C = align_up(w->B + nbk * E, 256);
    w->init = align_up(w->C + nbk * E, 256);
    w->dfin = align_up(w->init + nstk, 256);
    w->dinit = align_up(w->dfin + nstk, 256);
    w->dB = align_up(w->dinit + nstk, 256);
    w->dC = align_up(w->dB + nbk * 4, 256);
    w->dx = align_up(w->dC + nbk * 4, 256);
    w->ddt = align_up(w->dx + w->nsplit * align_up(nx * E, 256), 256);
    w->dA = align_up(w->ddt + w->nsplit * align_up(tokens * d.nheads * 4, 256), 256);
    w->dD = align_up(w->dA + (size_t)w->nsplit * d.nheads * 4, 256);
    w->total = align_up(w->dD + (size_t)w->nsplit * d.nheads * 4, 256);
    return true;
}

size_t bwd_ws_total(const ssd_dims_t &d, ssd_dtype_t io, bool varlen) {
    BwdSplitWs sw{};
    bwd_split_ws(d, io, varlen, &sw);
    return sw.nsplit > 1 ? sw.total : sw.inner.total;
}

// Runs the backward kernels on contiguous inputs whose state dim d.dstate is
// built (validation done by the caller).
ssd_status_t bwd_run(const ssd_dims_t &d, ssd_dtype_t io, const void *x, const float *dt, const float *A,
                     const void *B, const void *C, const float *D, const float *init_state,
                     const int32_t *cu_seqlens, const void *dy, const float *dfinal_state, void *dx, float *ddt,
                     float *dA, float *dB, float *dC, float *dD, float *dinit_state, char *ws, hipStream_t s) {
    BwdWs w{};
    bwd_ws(d, cu_seqlens != nullptr, &w);
    ssd::BwdPrepParams pp{};
    pp.cu_seqlens = cu_seqlens;
    pp.batch = d.batch;
    pp.seqlen = d.seqlen;
    pp.nseq = d.nseq;
    pp.seq_chunk_start = reinterpret_cast<int *>(ws + w.seqstart);
    pp.chunks = reinterpret_cast<int4 *>(ws + w.chunks);
    hipLaunchKernelGGL(ssd::ssd_bwd_prep_kernel, dim3(1), dim3(256), 0, s, pp);

    ssd::BwdParams p{};
    p.x = x;
    p.B = B;
    p.C = C;
    p.dy = dy;
    p.dt = dt;
    p.A = A;
    p.D = D;
    p.init_state = init_state;
    p.dfinal = dfinal_state;
    p.dx = dx;
    p.ddt = ddt;
    p.dB = dB;
    p.dC = dC;
    p.dinit = dinit_state;
    p.dA = dA;
    p.dD = dD;
    p.chunks = pp.chunks;
    p.seq_chunk_start = pp.seq_chunk_start;
    p.states = reinterpret_cast<float *>(ws + w.states);
    p.radj = reinterpret_cast<float *>(ws + w.radj);
    p.partA = reinterpret_cast<float *>(ws + w.partA);
    p.partD = reinterpret_cast<float *>(ws + w.partD);
    const KHeads kh = kernel_heads(d);
    p.H = kh.H;
    p.hsub = kh.hsub;
    p.G = d.ngroups;
    p.nseq = d.nseq;
    const unsigned units = (unsigned)d.nseq * (unsigned)kh.H;
    const bool ok = (io == SSD_BF16)
                        ? ssd::bwd_dispatch<ssd::bf16>(kh.P, d.dstate, p, units, (unsigned)w.max_chunks, true, s)
                        : ssd::bwd_dispatch<float>(kh.P, d.dstate, p, units, (unsigned)w.max_chunks, true, s);
    if (!ok) return SSD_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(ssd::ssd_bwd_reduce_kernel, dim3(d.nheads), dim3(256), 0, s, p);
    if (hipGetLastError() != hipSuccess) return SSD_ERR_HIP;
    return SSD_OK;
}

// Columns [c0, c0 + w) of `rows` rows of `pitch_src` bytes into a packed
// buffer (or back, with the pitches exchanged).
bool copy_cols(void *dst, size_t dpitch, const void *src, size_t spitch, size_t width, size_t rows, hipStream_t s) {
    if (rows == 0) return true;
    return hipMemcpy2DAsync(dst, dpitch, src, spitch, width, rows, hipMemcpyDeviceToDevice, s) == hipSuccess;
}
}  // namespace
}  // extern "C"

namespace ssd {
// Sums of the state-dim slices' terms, slice 0 first: dx (rounded once to the
// io dtype), ddt and dA; dD is slice 0's (it does not depend on the state dim).
template <typename IO>
__global__ __launch_bounds__(256) void ssd_bwd_combine_kernel(IO *dx, const IO *dxk, size_t nx, size_t px,
                                                              float *ddt, const float *ddtk, size_t nt, size_t pt,
                                                              float *dA, const float *dAk, float *dD,
                                                              const float *dDk, int H, int nsplit) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nx; i += stride) {
        float v = 0.f;
        for (int k = 0; k < nsplit; ++k) v += to_f32(dxk[k * px + i]);
        dx[i] = from_f32<IO>(v);
    }
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nt; i += stride) {
        float v = 0.f;
        for (int k = 0; k < nsplit; ++k) v += ddtk[k * pt + i];
        ddt[i] = v;
    }
    if (blockIdx.x == 0) {
        for (int h = threadIdx.x; h < H; h += blockDim.x) {
            float v = 0.f;
            for (int k = 0; k < nsplit; ++k) v += dAk[k * H + h];
            dA[h] = v;
            dD[h] = dDk[h];
        }
    }
}
}  // namespace ssd

extern "C" {

size_t ssd_chunk_scan_bwd_workspace_size(const ssd_dims_t *dims, ssd_dtype_t io) {
    if (!dims) return 0;
    if (bwd_shape_check(dims, io, true) != SSD_OK && bwd_shape_check(dims, io, false) != SSD_OK) return 0;
    const size_t a = bwd_ws_total(*dims, io, true), b = bwd_ws_total(*dims, io, false);
    return a > b ? a : b;
}

ssd_status_t ssd_chunk_scan_bwd(const ssd_dims_t *dims, ssd_dtype_t io, const void *x, const float *dt,
                                const float *A, const void *B, const void *C, const float *D,
                                const float *init_state, const int32_t *cu_seqlens, const void *dy,
                                const float *dfinal_state, void *dx, float *ddt, float *dA, float *dB, float *dC,
                                float *dD, float *dinit_state, void *workspace, size_t workspace_bytes,
                                void *stream) {
    const bool varlen = cu_seqlens != nullptr;
    ssd_status_t st = bwd_shape_check(dims, io, varlen);
    if (st != SSD_OK) return st;
    const ssd_dims_t &d = *dims;
    if (!x || !dt || !A || !B || !C || !dy || !dx || !ddt || !dA || !dB || !dC || !dD) return SSD_ERR_NULL_PTR;
    if (!workspace) return SSD_ERR_WORKSPACE;
    const void *al16[] = {x, dt, A, B, C, D, init_state, dy, dfinal_state, dx, ddt, dA, dB, dC, dD, dinit_state};
    for (const void *q : al16)
        if (q && !aligned(q, 16)) return SSD_ERR_ALIGNMENT;
    if (!aligned(workspace, 256)) return SSD_ERR_ALIGNMENT;
    if (cu_seqlens && !aligned(cu_seqlens, 4)) return SSD_ERR_ALIGNMENT;
    const size_t ws_total = bwd_ws_total(d, io, varlen);
    if (workspace_bytes < ws_total) return SSD_ERR_WORKSPACE;

    const size_t E = (io == SSD_BF16) ? 2 : 4;
    const size_t tokens = (size_t)d.batch * d.seqlen;
    const size_t nx = tokens * d.nheads * d.headdim, nbc = tokens * d.ngroups * d.dstate;
    const size_t nst = (size_t)d.nseq * d.nheads * d.headdim * d.dstate * 4;
    const Range ins[] = {rng(x, nx * E), rng(dt, tokens * d.nheads * 4), rng(A, (size_t)d.nheads * 4),
                         rng(B, nbc * E), rng(C, nbc * E), rng(D, D ? (size_t)d.nheads * 4 : 0),
                         rng(init_state, init_state ? nst : 0), rng(dy, nx * E),
                         rng(dfinal_state, dfinal_state ? nst : 0),
                         rng(cu_seqlens, varlen ? (size_t)(d.nseq + 1) * 4 : 0), rng(workspace, ws_total)};
    const Range outs[] = {rng(dx, nx * E), rng(ddt, tokens * d.nheads * 4), rng(dA, (size_t)d.nheads * 4),
                          rng(dB, nbc * 4), rng(dC, nbc * 4), rng(dD, (size_t)d.nheads * 4),
                          rng(dinit_state, dinit_state ? nst : 0)};
    for (size_t a = 0; a < sizeof(outs) / sizeof(outs[0]); ++a) {
        for (const Range &r : ins)
            if (overlap(outs[a], r)) return SSD_ERR_ALIAS;
        for (size_t b = a + 1; b < sizeof(outs) / sizeof(outs[0]); ++b)
            if (overlap(outs[a], outs[b])) return SSD_ERR_ALIAS;
    }

    char *ws = static_cast<char *>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = debug_check_cu_seqlens(cu_seqlens, d.nseq, d.seqlen, s);
    if (st != SSD_OK) return st;
    BwdSplitWs sw{};
    bwd_split_ws(d, io, varlen, &sw);
    if (sw.nsplit <= 1)
        return bwd_run(d, io, x, dt, A, B, C, D, init_state, cu_seqlens, dy, dfinal_state, dx, ddt, dA, dB, dC, dD,
                       dinit_state, ws, s);

    // state-dim slices of kn columns: copy the slice's B, C and states in,
    // run, copy its dB, dC and dinit columns out; dx, ddt and dA are summed
    ssd_dims_t dk = d;
    dk.dstate = sw.kn;
    const size_t kn = (size_t)sw.kn, N = (size_t)d.dstate;
    const size_t rows_bc = tokens * d.ngroups, rows_st = (size_t)d.nseq * d.nheads * d.headdim;
    const size_t px = align_up(nx * E, 256), pt = align_up(tokens * d.nheads * 4, 256);
    void *Bk = ws + sw.B, *Ck = ws + sw.C;
    float *ik = init_state ? reinterpret_cast<float *>(ws + sw.init) : nullptr;
    float *fk = dfinal_state ? reinterpret_cast<float *>(ws + sw.dfin) : nullptr;
    float *dik = dinit_state ? reinterpret_cast<float *>(ws + sw.dinit) : nullptr;
    float *dBk = reinterpret_cast<float *>(ws + sw.dB), *dCk = reinterpret_cast<float *>(ws + sw.dC);
    for (int k = 0; k < sw.nsplit; ++k) {
        const size_t c0 = (size_t)k * kn;
        bool ok = copy_cols(Bk, kn * E, static_cast<const char *>(B) + c0 * E, N * E, kn * E, rows_bc, s) &&
                  copy_cols(Ck, kn * E, static_cast<const char *>(C) + c0 * E, N * E, kn * E, rows_bc, s);
        if (ik) ok = ok && copy_cols(ik, kn * 4, init_state + c0, N * 4, kn * 4, rows_st, s);
        if (fk) ok = ok && copy_cols(fk, kn * 4, dfinal_state + c0, N * 4, kn * 4, rows_st, s);
        if (!ok) return SSD_ERR_HIP;
        st = bwd_run(dk, io, x, dt, A, Bk, Ck, k == 0 ? D : nullptr, ik, cu_seqlens, dy, fk, ws + sw.dx + k * px,
                     reinterpret_cast<float *>(ws + sw.ddt + k * pt), reinterpret_cast<float *>(ws + sw.dA) + k * d.nheads,
                     dBk, dCk, reinterpret_cast<float *>(ws + sw.dD) + k * d.nheads, dik, ws, s);
        if (st != SSD_OK) return st;
        ok = copy_cols(dB + c0, N * 4, dBk, kn * 4, kn * 4, rows_bc, s) &&
             copy_cols(dC + c0, N * 4, dCk, kn * 4, kn * 4, rows_bc, s);
        if (dik) ok = ok && copy_cols(dinit_state + c0, N * 4, dik, kn * 4, kn * 4, rows_st, s);
        if (!ok) return SSD_ERR_HIP;
    }
    const size_t blocks = (nx + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 4096 ? (blocks > 0 ? blocks : 1) : 4096);
    if (io == SSD_BF16)
        hipLaunchKernelGGL(ssd::ssd_bwd_combine_kernel<ssd::bf16>, dim3(grid), dim3(256), 0, s,
                           static_cast<ssd::bf16 *>(dx), reinterpret_cast<const ssd::bf16 *>(ws + sw.dx), nx,
                           px / E, ddt, reinterpret_cast<const float *>(ws + sw.ddt), tokens * d.nheads, pt / 4, dA,
                           reinterpret_cast<const float *>(ws + sw.dA), dD,
                           reinterpret_cast<const float *>(ws + sw.dD), d.nheads, sw.nsplit);
    else
        hipLaunchKernelGGL(ssd::ssd_bwd_combine_kernel<float>, dim3(grid), dim3(256), 0, s, static_cast<float *>(dx),
                           reinterpret_cast<const float *>(ws + sw.dx), nx, px / E, ddt,
                           reinterpret_cast<const float *>(ws + sw.ddt), tokens * d.nheads, pt / 4, dA,
                           reinterpret_cast<const float *>(ws + sw.dA), dD,
                           reinterpret_cast<const float *>(ws + sw.dD), d.nheads, sw.nsplit);
    if (hipGetLastError() != hipSuccess) return SSD_ERR_HIP;
    return SSD_OK;
}

}  // extern "C"

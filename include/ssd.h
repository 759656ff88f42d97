/*
 * ssd.h -- C ABI of the MI355X (gfx950) SSD layer library, libssd.so.
 *
 * The layer is the selective state-space recurrence with a scalar decay per
 * head, which the Mamba-2 papers call structured state-space duality (SSD).
 * For every sequence, head h (group g = h / (nheads/ngroups)) and token t:
 *
 *     abar_t = exp(dt[t,h] * A[h])
 *     h_t    = abar_t * h_{t-1} + dt[t,h] * x[t,h,:] (outer) B[t,g,:]     (P x N)
 *     y[t,h] = h_t * C[t,g,:] + D[h] * x[t,h,:]
 *
 * Sources (cited by page title and section):
 *   - "Mamba-2는 왜 Transformer와 닮았는가: SSD로 다시 읽는 SSM" (bdev.io), the
 *     problem section: the recurrence h_t = A_t h_{t-1} + B_t x_t,
 *     y_t = C_t^T h_t.
 *   - "20.1 상태 공간 모델 (SSM)" textbook chapter (sungeuns.github.io),
 *     section 1: zero-order-hold Abar = exp(dt A) and Bbar ~= dt B, skip D;
 *     section 3: A restricted to a scalar times identity (one scalar per head);
 *     section 5: the state is updated before the output is read out.
 *   - "Transformers are SSMs Review" (dimensionstp.github.io), section
 *     3-2(4): the chunked SSD algorithm (quadratic masked form inside a chunk,
 *     chunk-boundary states passed between chunks); section 3-2(6): packed
 *     variable-length batches cut the state at sequence boundaries.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless noted, row-major and contiguous.
 *     The caller owns every buffer; the library allocates nothing, keeps no
 *     mutable global state and is reentrant.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and
 *     the call returns before it completes.  Asynchronous device faults show
 *     up at the caller's next synchronisation.
 *   - Arguments are validated synchronously before anything is launched; an
 *     invalid call returns a status and launches nothing.  No C++ exception
 *     crosses the ABI.
 *   - Preconditions that are documented but not checked on the host: inputs
 *     are finite; cu_seqlens[0] == 0, cu_seqlens is non-decreasing and its
 *     last entry is seqlen.  Non-finite values stay inside their own sequence.
 *     The forward's schedule kernel checks cu_seqlens on the device and, when
 *     it is broken, processes nothing (ssd_chunk_scan_fwd_check reports it).
 *   - With the environment variable SSD_DEBUG_VALIDATE=1, every entry point
 *     that takes cu_seqlens copies it to the host first (this synchronises
 *     `stream`, so not under graph capture) and returns SSD_ERR_SHAPE,
 *     launching nothing, when it breaks the precondition above.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 5

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL_PTR = 1,     /* a required pointer is NULL                         */
    SSD_ERR_SHAPE = 2,        /* a dimension is <= 0 or inconsistent                 */
    SSD_ERR_DTYPE = 3,        /* io dtype is not SSD_F32 or SSD_BF16                 */
    SSD_ERR_UNSUPPORTED = 4,  /* headdim/dstate/chunk_len combination not built      */
    SSD_ERR_ALIGNMENT = 5,    /* a pointer is not 16-byte aligned (workspace: 256)   */
    SSD_ERR_ALIAS = 6,        /* an output overlaps an input it must not overlap     */
    SSD_ERR_WORKSPACE = 7,    /* workspace NULL or smaller than the size query says  */
    SSD_ERR_HIP = 8,          /* the HIP runtime reported an error at launch         */
    SSD_ERR_DEVICE = 9,       /* a kernel reported an internal failure (see below)   */
    SSD_STATUS_MAX_ENUM = 0x7fffffff  /* not a status: every value in [0, 2^31) is in range */
} ssd_status_t;

/* dtype of x, B, C, y.  The last enumerator is not a dtype: it keeps every
 * value in [0, 2^31) in the type's range, so an invalid value passed by a
 * caller is rejected (SSD_ERR_DTYPE) rather than being undefined. */
typedef enum { SSD_F32 = 0, SSD_BF16 = 1, SSD_DTYPE_MAX_ENUM = 0x7fffffff } ssd_dtype_t;

typedef struct {
    int32_t batch;    /* dense batch size; 1 for a packed varlen batch               */
    int32_t seqlen;   /* tokens per batch row (varlen: total packed tokens)          */
    int32_t nheads;   /* H                                                           */
    int32_t headdim;  /* P, channels per head                                        */
    int32_t dstate;   /* N, state size per channel                                   */
    int32_t ngroups;  /* G, groups sharing B and C; nheads % ngroups == 0            */
    int32_t nseq;     /* number of sequences: == batch when cu_seqlens is NULL       */
} ssd_dims_t;

/*
 * Optional step-size preprocessing, applied on the device before dt is used.
 * The selective step size of the "20.1 상태 공간 모델 (SSM)" textbook chapter,
 * section 2, is the softplus of a linear projection of the input; dt_bias is
 * that projection's bias, one value per head.  Per token t and head h:
 *     v  = dt[t, h] + (dt_bias ? dt_bias[h] : 0)
 *     v  = softplus ? log(1 + exp(v)) : v
 *     dt = min(max(v, dt_min), dt_max)
 * (tokens beyond a sequence's end are not touched).  A NULL options pointer
 * uses dt as given.  dt_min <= dt_max is required (NaN bounds are rejected);
 * -INFINITY and INFINITY disable the clamp.
 *   dt_bias   [nheads] fp32 device pointer, or NULL
 */
typedef struct {
    const float *dt_bias;
    int32_t softplus;   /* nonzero: apply the softplus                          */
    float dt_min;       /* lower clamp after the softplus                       */
    float dt_max;       /* upper clamp after the softplus                       */
} ssd_dt_opts_t;

/* Human-readable name of a status code (static storage, never NULL). */
const char *ssd_status_string(ssd_status_t status);

/* SSD_ABI_VERSION of the built library. */
int32_t ssd_abi_version(void);

/*
 * Bytes of device workspace ssd_chunk_scan_fwd needs for these dimensions,
 * chunk length and io dtype, or 0 when the arguments are invalid.  The
 * workspace holds the chunk schedule, per-(sequence, head) progress flags and
 * the fp32 chunk-boundary states; it needs no initialisation by the caller.
 */
size_t ssd_chunk_scan_fwd_workspace_size(const ssd_dims_t *dims, int32_t chunk_len,
                                         ssd_dtype_t io_dtype);

/*
 * Chunked SSD forward pass (the chunked algorithm of "Transformers are SSMs
 * Review", section 3-2(4)): per chunk of chunk_len tokens the output is the
 * masked quadratic form (C B^T o L) dt x, plus the incoming chunk-boundary
 * state read out through C, plus D x; the boundary states are passed from
 * chunk to chunk in fp32.  The result equals the recurrence above; only the
 * evaluation order (and so the rounding) differs, and it does not depend on
 * chunk_len beyond rounding.
 *
 *   dims        host pointer.  Dense batch: cu_seqlens == NULL, nseq == batch.
 *               Packed varlen: batch == 1, cu_seqlens != NULL, nseq >= 1.
 *   io_dtype    dtype of x, B, C and y.  Arithmetic: fp32 accumulation and
 *               state; SSD_BF16 contractions run on bf16 MFMA, SSD_F32 on
 *               fp32 MFMA.
 *   chunk_len   64, 128 or 256.
 *   x           [batch, seqlen, nheads, headdim]  io
 *   dt          [batch, seqlen, nheads] fp32, the final (positive) step size
 *   A           [nheads] fp32, the scalar decay rate per head (expected <= 0;
 *               0 is allowed and gives linear attention)
 *   B, C        [batch, seqlen, ngroups, dstate]  io
 *   D           [nheads] fp32, or NULL for no skip term
 *   init_state  [nseq, nheads, headdim, dstate] fp32, or NULL for zeros.
 *               It may be the same buffer as final_state (in-place resume).
 *   cu_seqlens  [nseq + 1] int32 device offsets of the packed sequences, or
 *               NULL.  The state restarts from init_state (or zero) at every
 *               sequence start.  nseq <= 65536.
 *   y           [batch, seqlen, nheads, headdim] io, output; must not overlap
 *               any input.
 *   final_state [nseq, nheads, headdim, dstate] fp32 output, or NULL.
 *   workspace   device buffer of at least workspace_bytes >=
 *               ssd_chunk_scan_fwd_workspace_size(...) bytes, 256-byte
 *               aligned, not used by another call in flight.
 *   stream      hipStream_t, or NULL for the default stream.
 *
 * Supported sizes: headdim in {16, 32, 64, 128}; dstate in {16, 32, 64, 128,
 * 256}; chunk_len in {64, 128, 256}, every combination, both io dtypes.
 * Head dim 128 runs as two 64-channel halves (each state row depends only on
 * its own channel).  Where the tiles of chunk_len tokens do not fit in the
 * 160 KB of LDS of a gfx950 compute unit (bf16: dstate 256 with chunk_len
 * 256 and headdim >= 32; fp32: headdim >= 64 with chunk_len 256, and some
 * larger shapes at 128), the kernel runs the largest shorter chunk that fits
 * (at least 64 tokens): chunking only orders the evaluation, so the result is
 * the same up to rounding.  Other sizes return SSD_ERR_UNSUPPORTED; so
 * that one chunk of x spans less than 2^30 bytes, nheads * headdim must stay
 * below 2^20 (else SSD_ERR_SHAPE).
 * x, y, B, C, dt, D and the states must be 16-byte aligned.
 */
ssd_status_t ssd_chunk_scan_fwd(const ssd_dims_t *dims, ssd_dtype_t io_dtype,
                                int32_t chunk_len,
                                const void *x, const float *dt, const float *A,
                                const void *B, const void *C, const float *D,
                                const float *init_state, const int32_t *cu_seqlens,
                                void *y, float *final_state,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * ssd_chunk_scan_fwd with step-size preprocessing (see ssd_dt_opts_t): `dt`
 * then holds the raw projection output.  dt_opts may be NULL (identical to
 * ssd_chunk_scan_fwd).  dt_bias must not overlap y or final_state.
 */
ssd_status_t ssd_chunk_scan_fwd_ex(const ssd_dims_t *dims, ssd_dtype_t io_dtype,
                                   int32_t chunk_len, const ssd_dt_opts_t *dt_opts,
                                   const void *x, const float *dt, const float *A,
                                   const void *B, const void *C, const float *D,
                                   const float *init_state, const int32_t *cu_seqlens,
                                   void *y, float *final_state,
                                   void *workspace, size_t workspace_bytes, void *stream);

/* Size of the device scratch array behind ssd_chunk_scan_fwd_noalloc. */
#define SSD_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * ssd_chunk_scan_fwd_ex that allocates nothing and takes no workspace: for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments,
 * semantics, outputs and status codes as ssd_chunk_scan_fwd_ex, minus the
 * workspace.  The workspace it would need (ssd_chunk_scan_fwd_workspace_size,
 * less the boundary-state part when final_state is given) lives in a
 * library-owned device array of SSD_NOALLOC_SCRATCH_BYTES (32 MiB), one per
 * device, held from the first call on that device until the process ends.
 * Dimensions whose workspace exceeds it return SSD_ERR_WORKSPACE and launch
 * nothing.  The schedule kernel clears what must start at zero on every call.
 * Every call on one device shares that device's array: calls that overlap in
 * time on one device (different streams, different threads) race and give
 * undefined results; serialise them.  There is no check call for this entry
 * point (the failure word sits in the shared array).
 */
ssd_status_t ssd_chunk_scan_fwd_noalloc(const ssd_dims_t *dims, ssd_dtype_t io_dtype,
                                        int32_t chunk_len, const ssd_dt_opts_t *dt_opts,
                                        const void *x, const float *dt, const float *A,
                                        const void *B, const void *C, const float *D,
                                        const float *init_state, const int32_t *cu_seqlens,
                                        void *y, float *final_state, void *stream);

/*
 * Checks a forward call after the fact (synchronises `stream`, then reads the
 * workspace header).  Returns
 *   SSD_OK          the call ran to completion;
 *   SSD_ERR_SHAPE   cu_seqlens broke its precondition (the kernel then
 *                   processed no chunk: y and final_state were not written);
 *   SSD_ERR_DEVICE  a chunk waited too long for its predecessor's state, or
 *                   some accelerator complex (XCD) never drained its list of
 *                   work items (every chain of chunks is bound to one XCD);
 *                   the outputs of that call are then invalid;
 *   SSD_ERR_HIP / SSD_ERR_WORKSPACE on a runtime error or a NULL workspace.
 * Meant for tests and diagnostics; the forward call itself does not wait.
 */
ssd_status_t ssd_chunk_scan_fwd_check(const void *workspace, void *stream);

/*
 * One recurrent decode step for a single new token per sequence, updating
 * the state in place (constant-size state per generated token, "Mamba-2는
 * 왜 Transformer와 닮았는가", the problem section):
 *     state = exp(dt A) state + dt x (outer) B;   y = state C + D x.
 *
 *   dims     host pointer; batch, nheads, headdim, dstate, ngroups are used
 *            (seqlen and nseq are ignored).
 *   state    [batch, nheads, headdim, dstate] fp32, read and written in place
 *   x        [batch, nheads, headdim] io
 *   dt       [batch, nheads] fp32
 *   A, D     [nheads] fp32 (D may be NULL)
 *   B, C     [batch, ngroups, dstate] io
 *   y        [batch, nheads, headdim] io output; must not overlap the inputs.
 *
 * Supported sizes: headdim >= 1, dstate in {16, 32, 64, 128, 256}.
 */
ssd_status_t ssd_decode_step(const ssd_dims_t *dims, ssd_dtype_t io_dtype,
                             float *state, const void *x, const float *dt,
                             const float *A, const void *B, const void *C,
                             const float *D, void *y, void *stream);

/*
 * ssd_decode_step with step-size preprocessing (see ssd_dt_opts_t); dt_opts
 * may be NULL.  dt_bias must not overlap y or state.
 */
ssd_status_t ssd_decode_step_ex(const ssd_dims_t *dims, ssd_dtype_t io_dtype,
                                const ssd_dt_opts_t *dt_opts, float *state,
                                const void *x, const float *dt, const float *A,
                                const void *B, const void *C, const float *D,
                                void *y, void *stream);

/*
 * Block prologue: the short causal convolution and activation that the Mamba
 * block applies to one projected branch before the selective SSM
 * ("Mamba - Linear-Time Sequence Modeling with Selective State Spaces" review,
 * feghi.github.io, section 5, the block figure read bottom to top), here over
 * the fused x | B | C projection of the Mamba-2 block ("Transformers are SSMs
 * Review", section 3-2, item 5: the data-dependent projections are made in
 * parallel at the start of the block).  Depthwise, per sequence:
 *
 *     u[t, c]   = the channel-c input of token t of the sequence, preceded by
 *                 the width-1 rows of conv_state (zeros when conv_state is NULL)
 *     out[t, c] = act(bias[c] + sum_{k<width} weight[c, k] * u[t - (width-1) + k, c])
 *
 * (the last tap multiplies the current token), act = SiLU (v / (1 + e^-v))
 * when `silu` is nonzero, else the identity.  fp32 arithmetic, io output
 * rounded to nearest even.
 *
 *   dims        host pointer; batch, seqlen, nheads, headdim, dstate, ngroups,
 *               nseq as for ssd_chunk_scan_fwd (nseq == batch for a dense
 *               batch; batch == 1 with cu_seqlens).
 *   width       number of taps, 1..4.
 *   xbc         [batch, seqlen, channels] io, channels = nheads*headdim +
 *               2*ngroups*dstate in the order x | B | C.
 *   weight      [channels, width] fp32;  bias [channels] fp32 or NULL.
 *   conv_state  [nseq, width-1, channels] io or NULL: the width-1 inputs that
 *               precede each sequence (a previous segment's conv_state_out).
 *   cu_seqlens  as for ssd_chunk_scan_fwd (device int32, or NULL).
 *   x           [batch, seqlen, nheads, headdim] io output (channels x);
 *   B, C        [batch, seqlen, ngroups, dstate] io outputs (channels B, C):
 *               the layouts ssd_chunk_scan_fwd reads.
 *   conv_state_out  [nseq, width-1, channels] io or NULL: each sequence's last
 *               width-1 rows of u (its initial state rows where it is shorter,
 *               the initial state itself for an empty packed sequence).
 *
 * Supported: headdim and dstate multiples of 8.  Pointers 16-byte aligned
 * (cu_seqlens 4).  The outputs must not overlap each other or any input
 * (conv_state_out must not be conv_state: SSD_ERR_ALIAS).
 */
ssd_status_t ssd_causal_conv1d_fwd(const ssd_dims_t *dims, ssd_dtype_t io_dtype, int32_t width,
                                   const void *xbc, const float *weight, const float *bias,
                                   int32_t silu, const void *conv_state, const int32_t *cu_seqlens,
                                   void *x, void *B, void *C, void *conv_state_out, void *stream);

/*
 * Block epilogue: the multiplicative gate of the Mamba block's second branch
 * (feghi.github.io review, section 5) with the NormFormer-style extra
 * normalization of Mamba-2 ("Transformers are SSMs Review", section 3-2,
 * item 5), as RMSNorm over groups of `group_size` consecutive channels:
 *
 *     rms(v) = sqrt(mean over the group of v^2 + eps)
 *     norm_before_gate == 0:  out = v / rms(v) * weight,  v = y * silu(z)
 *     norm_before_gate != 0:  out = y / rms(y) * weight * silu(z)
 *
 * fp32 arithmetic, io output rounded to nearest even.
 *
 *   rows        number of token rows (batch * seqlen).
 *   dim         channels per row (nheads * headdim);  group_size divides dim.
 *   y           [rows, dim] io (the SSD output);  z [rows, dim] io gate input,
 *               or NULL for a plain RMSNorm.
 *   weight      [dim] fp32.   eps >= 0 and finite (eps = 0 with an all-zero
 *               group gives NaN, as the formula does).
 *   out         [rows, dim] io output; may be y or z itself (in place), must
 *               not overlap them otherwise, nor weight.
 *
 * Supported: group_size a multiple of 8, at most 8192 channels (bf16) or
 * 4096 (fp32).  Pointers 16-byte aligned.
 */
ssd_status_t ssd_gated_rmsnorm_fwd(int64_t rows, int32_t dim, int32_t group_size, ssd_dtype_t io_dtype,
                                   const void *y, const void *z, const float *weight, float eps,
                                   int32_t norm_before_gate, void *out, void *stream);

/*
 * Backward pass of ssd_chunk_scan_fwd: the gradients of
 *     L = <dy, y> + <dfinal_state, final_state>
 * with respect to x, dt, A, B, C, D and init_state, through the same chunked
 * evaluation ("Transformers are SSMs Review", section 3-2(4)); the pages
 * print no backward pass, so this is reverse-mode differentiation of that
 * forward (the chunk-boundary states are recomputed, and the state gradients
 * are chained backwards over the chunks; 64-token chunks internally, which
 * changes only the rounding).
 *
 *   dims, io_dtype, x, dt, A, B, C, D, init_state, cu_seqlens: as for the
 *               forward call whose gradient is wanted (dt is the final step
 *               size; chain any preprocessing through the caller).
 *   dy          [batch, seqlen, nheads, headdim] io
 *   dfinal_state [nseq, nheads, headdim, dstate] fp32, or NULL (zero)
 *   dx          [batch, seqlen, nheads, headdim] io output
 *   ddt         [batch, seqlen, nheads] fp32 output
 *   dA, dD      [nheads] fp32 outputs (dD also when D is NULL)
 *   dB, dC      [batch, seqlen, ngroups, dstate] fp32 outputs, summed over
 *               the heads of each group
 *   dinit_state [nseq, nheads, headdim, dstate] fp32 output, or NULL
 *   workspace   >= ssd_chunk_scan_bwd_workspace_size(dims, io_dtype) bytes,
 *               256-byte aligned, not used by another call in flight (holds
 *               every chunk-boundary state and state gradient: about
 *               2 * tokens/64 * nheads * headdim * dstate * 4 bytes; for a
 *               state dim run in slices, see below, that of one slice plus
 *               the slices' inputs and dx, ddt terms).
 *
 * Deterministic (fixed reduction orders, no atomics).  Supported: headdim in
 * {16, 32, 64, 128}, dstate in {16, 32, 64, 128, 256}, both io dtypes; other
 * sizes return SSD_ERR_UNSUPPORTED.  Head dim 128 runs as two kernel heads of
 * 64 channels (every state row depends only on its own channel of x), whose
 * ddt, dA and dD terms are added in a fixed order.  State dims beyond the
 * kernels' (bf16: 256; fp32: 128 and 256) run once per slice of 128 (bf16) or
 * 64 (fp32) state columns: every state column evolves on its own and y is a
 * sum over them, so each slice gives its columns of dB, dC and dinit and one
 * term of dx, ddt and dA, added slice by slice (dx rounded to the io dtype
 * once); the slices' B, C and states are copied through the workspace.
 * Outputs must not overlap each other, the inputs or the workspace.
 */
size_t ssd_chunk_scan_bwd_workspace_size(const ssd_dims_t *dims, ssd_dtype_t io_dtype);

ssd_status_t ssd_chunk_scan_bwd(const ssd_dims_t *dims, ssd_dtype_t io_dtype,
                                const void *x, const float *dt, const float *A,
                                const void *B, const void *C, const float *D,
                                const float *init_state, const int32_t *cu_seqlens,
                                const void *dy, const float *dfinal_state,
                                void *dx, float *ddt, float *dA, float *dB, float *dC,
                                float *dD, float *dinit_state,
                                void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */

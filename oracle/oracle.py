"""fp64 CPU oracle for the SSD layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The product library never links, loads
or calls it, and it shares no code with the HIP path.

It wraps ``ssd_oracle.c`` (plain C, fp64, sequential recurrence; see that
file's header for the passages of the pages it follows) through ctypes.
Inputs of any float dtype are upcast exactly to float64 (bf16 and fp32 values
are exactly representable in fp64).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB = os.path.join(_HERE, "libssd_oracle.so")
_lib = None

_F64P = ctypes.POINTER(ctypes.c_double)
_I64P = ctypes.POINTER(ctypes.c_int64)
_U8P = ctypes.POINTER(ctypes.c_uint8)


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (IEEE fp64: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-shared", "-fPIC", _SRC, "-o", tmp, "-lm",
        ])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.ssd_oracle_fwd.restype = ctypes.c_int
        lib.ssd_oracle_fwd.argtypes = [
            ctypes.c_int64, _I64P, _I64P,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            _F64P, _F64P, _F64P, _F64P, _F64P, _F64P, _F64P, _U8P,
            _F64P, _F64P, ctypes.c_int,
        ]
        lib.ssd_oracle_decode.restype = ctypes.c_int
        lib.ssd_oracle_decode.argtypes = [
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            _F64P, _F64P, _F64P, _F64P, _F64P, _F64P, _F64P, _F64P, ctypes.c_int,
        ]
        _lib = lib
    return _lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a, typ=_F64P):
    return None if a is None else a.ctypes.data_as(typ)


def ssd_fwd(x, dt, A, B, C, D=None, init_state=None, cu_seqlens=None,
            unit_mask=None, nthreads: int = 0):
    """Sequential fp64 SSD forward.

    Dense batch: x [b, L, H, P], dt [b, L, H], B/C [b, L, G, N].
    Packed varlen: pass ``cu_seqlens`` (length nseq+1) with b == 1.
    ``unit_mask`` [nseq, H] (bool) restricts the work to some (sequence, head)
    pairs; outputs of skipped pairs are left at zero.
    Returns (y [b, L, H, P] float64, final_state [nseq, H, P, N] float64).
    """
    x = _f64(x); dt = _f64(dt); A = _f64(A); B = _f64(B); C = _f64(C)
    D = _f64(D); init_state = _f64(init_state)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (b, L, H) and B.shape == (b, L, G, N) and C.shape == B.shape
    assert A.shape == (H,)
    if cu_seqlens is None:
        nseq = b
        starts = np.arange(b, dtype=np.int64) * L
        lens = np.full(b, L, dtype=np.int64)
    else:
        assert b == 1
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        nseq = cu.size - 1
        starts = np.ascontiguousarray(cu[:-1])
        lens = np.ascontiguousarray(cu[1:] - cu[:-1])
        assert cu[0] == 0 and cu[-1] == L and np.all(lens >= 0)
    if init_state is not None:
        assert init_state.shape == (nseq, H, P, N)
    mask = None
    if unit_mask is not None:
        mask = np.ascontiguousarray(np.asarray(unit_mask, dtype=np.uint8).reshape(nseq * H))
    y = np.zeros((b, L, H, P), dtype=np.float64)
    fin = np.zeros((nseq, H, P, N), dtype=np.float64)
    rc = _load().ssd_oracle_fwd(
        nseq, _ptr(starts, _I64P), _ptr(lens, _I64P), H, P, N, G,
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init_state),
        _ptr(mask, _U8P), _ptr(y), _ptr(fin), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"ssd_oracle_fwd failed with code {rc}")
    return y, fin


def ssd_decode(state, x, dt, A, B, C, D=None, nthreads: int = 0):
    """One fp64 recurrent step.  state [b, H, P, N]; x [b, H, P]; dt [b, H];
    B/C [b, G, N].  Returns (y [b, H, P], new_state [b, H, P, N]); the input
    array is not modified."""
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    x = _f64(x); dt = _f64(dt); A = _f64(A); B = _f64(B); C = _f64(C); D = _f64(D)
    b, H, P, N = st.shape
    G = B.shape[1]
    assert x.shape == (b, H, P) and dt.shape == (b, H) and B.shape == (b, G, N)
    y = np.zeros((b, H, P), dtype=np.float64)
    rc = _load().ssd_oracle_decode(b, H, P, N, G, _ptr(st), _ptr(x), _ptr(dt), _ptr(A),
                                   _ptr(B), _ptr(C), _ptr(D), _ptr(y), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"ssd_oracle_decode failed with code {rc}")
    return y, st


def dt_preprocess(dt_raw, dt_bias=None, softplus: bool = False, dt_min: float = -np.inf,
                  dt_max: float = np.inf):
    """Step-size preprocessing in fp64: clamp(softplus(dt_raw + dt_bias)).

    The "20.1 상태 공간 모델 (SSM)" textbook chapter, section 2, makes the step
    size the softplus of a linear projection of the input; dt_bias is that
    projection's bias, one value per head (the last axis of dt_raw).  The clamp
    bounds are applied after the softplus.  softplus(v) = log(1 + exp(v)) is
    evaluated as max(v, 0) + log1p(exp(-|v|)), which does not overflow.
    """
    v = np.asarray(dt_raw, dtype=np.float64)
    if dt_bias is not None:
        v = v + np.asarray(dt_bias, dtype=np.float64)
    if softplus:
        v = np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))
    return np.minimum(np.maximum(v, dt_min), dt_max)


# --------------------------------------------------------------------------
# Block prologue and epilogue around the SSD layer.
#
# The Mamba block of the feghi.github.io Mamba review (section 5, the block
# figure read bottom to top) sends one projected branch through a short causal
# convolution and an activation before the selective SSM, while the other
# branch becomes a multiplicative gate on the SSM output; the Mamba-2 review
# (section 3-2, item 5) adds a NormFormer-style extra normalization there.  The
# pages name neither the activation, the convolution width nor the norm; the
# readings used here (SiLU, a depthwise causal convolution whose last tap
# multiplies the current token, RMSNorm with a per-channel weight over groups of
# channels) are listed with the other readings of the pages in the design notes.

def silu(v):
    """v * logistic(v) in fp64, with logistic(v) = (1 + tanh(v / 2)) / 2 (no overflow)."""
    v = np.asarray(v, dtype=np.float64)
    return v * 0.5 * (1.0 + np.tanh(0.5 * v))


def causal_conv1d(xbc, weight, bias=None, activation: bool = False, conv_state=None, cu_seqlens=None):
    """Depthwise causal convolution over the token axis, per sequence, in fp64.

    xbc [batch, seqlen, channels]; weight [channels, width]; bias [channels] or
    None.  For a token t of a sequence starting at token a,
        out[t, c] = bias[c] + sum_k weight[c, k] * u[t - (width - 1) + k, c],
    where u is the sequence's input, preceded by the width-1 rows of
    conv_state[s] (the previous segment's last inputs), or by zeros without a
    state.  SiLU is applied after the bias when `activation`.  With cu_seqlens
    (int [nseq + 1]) the batch must be 1 and each [cu[s], cu[s+1]) is one
    sequence; otherwise each batch row is one.  Returns (out, final_state) with
    final_state [nseq, width - 1, channels]: each sequence's last width-1 rows
    of u (taken from its initial state where the sequence is shorter).
    """
    x = np.asarray(xbc, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    b_, L, Cc = x.shape
    W = w.shape[1]
    assert w.shape[0] == Cc and W >= 1
    if cu_seqlens is not None:
        assert b_ == 1
        cu = [int(v) for v in np.asarray(cu_seqlens)]
        spans = [(0, cu[s], cu[s + 1]) for s in range(len(cu) - 1)]
    else:
        spans = [(bi, 0, L) for bi in range(b_)]
    nseq = len(spans)
    out = np.zeros_like(x)
    final = np.zeros((nseq, W - 1, Cc))
    for s, (bi, a, e) in enumerate(spans):
        head = (np.zeros((W - 1, Cc)) if conv_state is None
                else np.asarray(conv_state, dtype=np.float64)[s])
        u = np.concatenate([head, x[bi, a:e]], axis=0)      # u[W-1 + i] is token a + i
        for i in range(e - a):
            acc = np.zeros(Cc) if bias is None else np.asarray(bias, dtype=np.float64).copy()
            for k in range(W):
                acc = acc + w[:, k] * u[i + k]
            out[bi, a + i] = silu(acc) if activation else acc
        if W > 1:
            final[s] = u[len(u) - (W - 1):]
    return out, final


def gated_rmsnorm(y, z, weight, eps: float, group_size=None, norm_before_gate: bool = False):
    """Gated RMSNorm over the last axis, in fp64, per group of `group_size`
    consecutive channels (the whole axis when None):
        rms(v) = sqrt(mean over the group of v^2 + eps),
        norm_before_gate:  out = y / rms(y) * weight * silu(z)
        otherwise:         out = v / rms(v) * weight,  v = y * silu(z).
    z may be None (no gate).
    """
    y = np.asarray(y, dtype=np.float64)
    D = y.shape[-1]
    gs = D if group_size is None else int(group_size)
    assert D % gs == 0
    g = np.ones_like(y) if z is None else silu(z)
    v = y if norm_before_gate else y * g
    vg = v.reshape(y.shape[:-1] + (D // gs, gs))
    rms = np.sqrt(np.mean(vg * vg, axis=-1, keepdims=True) + eps)
    out = (vg / rms).reshape(y.shape) * np.asarray(weight, dtype=np.float64)
    return out * g if norm_before_gate else out


# --------------------------------------------------------------------------
# Backward pass.
#
# The gradient of a scalar loss through the recurrence of ssd_fwd (bdev.io,
# problem section: h_t = Abar_t h_{t-1} + Bbar_t x_t, y_t = C_t^T h_t; the
# textbook chapter's section 1 and 3 discretisation with a scalar decay per
# head), written out as the adjoint recurrence that runs backwards over the
# tokens: with g_t = dL/dh_t,
#     g_t      = dy_t C_t^T + Abar_{t+1} g_{t+1}      (g_last = dy_last C^T + dfinal)
#     dx_t     = D dy_t + dt_t g_t B_t
#     dB_t    += dt_t g_t^T x_t            (summed over the heads of B's group)
#     dC_t    += h_t^T dy_t                (likewise)
#     q_t      = <g_t, Abar_t h_{t-1}>     (Frobenius product)
#     ddt_t    = x_t^T g_t B_t + A q_t
#     dA      += dt_t q_t
#     dD      += dy_t . x_t
#     dinit    = Abar_first g_first
# The pages do not print a backward pass; this is reverse-mode
# differentiation of the forward above, pinned against finite differences of
# the C oracle in the tests.

def ssd_bwd(x, dt, A, B, C, dy, D=None, init_state=None, cu_seqlens=None, dfinal=None, unit_mask=None):
    """fp64 gradients of L = <dy, y> + <dfinal, final_state> for y, final_state
    = ssd_fwd(x, dt, A, B, C, D, init_state, cu_seqlens).

    Shapes as for ssd_fwd; dy like y, dfinal like final_state (or None).
    Returns a dict with dx [b, L, H, P], ddt [b, L, H], dA [H], dB and dC
    [b, L, G, N], dD [H] and dinit [nseq, H, P, N], plus dA_abs [H]: the sum
    of the absolute values of dA's per-token terms dt_t <dL/dh_t, abar_t
    h_{t-1}>, the scale against which dA's rounding error is measured (its
    terms can cancel).  ``unit_mask`` [nseq, H]
    (bool) restricts the work to some (sequence, head) pairs: the other pairs'
    gradients stay zero, and dB, dC, dA, dD sum the chosen pairs only."""
    x = _f64(x); dt = _f64(dt); A = _f64(A); B = _f64(B); C = _f64(C); dy = _f64(dy)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    Dv = np.zeros(H) if D is None else _f64(D)
    if cu_seqlens is None:
        spans = [(bi, 0, L) for bi in range(b)]
    else:
        assert b == 1
        cu = [int(v) for v in np.asarray(cu_seqlens)]
        spans = [(0, cu[s], cu[s + 1]) for s in range(len(cu) - 1)]
    nseq = len(spans)
    init = np.zeros((nseq, H, P, N)) if init_state is None else _f64(init_state)
    dfin = np.zeros((nseq, H, P, N)) if dfinal is None else _f64(dfinal)
    out = dict(dx=np.zeros_like(x), ddt=np.zeros_like(dt), dA=np.zeros(H), dB=np.zeros_like(B),
               dC=np.zeros_like(C), dD=np.zeros(H), dinit=np.zeros((nseq, H, P, N)), dA_abs=np.zeros(H))
    for s, (bi, a, e) in enumerate(spans):
        for h in range(H):
            if unit_mask is not None and not unit_mask[s][h]:
                continue
            g_ = h // hpg
            # forward, keeping every state
            hs = np.zeros((e - a + 1, P, N))
            hs[0] = init[s, h]
            for i, t in enumerate(range(a, e)):
                abar = np.exp(dt[bi, t, h] * A[h])
                hs[i + 1] = abar * hs[i] + dt[bi, t, h] * np.outer(x[bi, t, h], B[bi, t, g_])
            # backward
            g = dfin[s, h].copy()
            for i in range(e - a - 1, -1, -1):
                t = a + i
                abar = np.exp(dt[bi, t, h] * A[h])
                g = g + np.outer(dy[bi, t, h], C[bi, t, g_])          # dL/dh_t
                out["dC"][bi, t, g_] += hs[i + 1].T @ dy[bi, t, h]
                gB = g @ B[bi, t, g_]
                out["dx"][bi, t, h] += Dv[h] * dy[bi, t, h] + dt[bi, t, h] * gB
                out["dB"][bi, t, g_] += dt[bi, t, h] * (g.T @ x[bi, t, h])
                q = float(np.sum(g * (abar * hs[i])))
                out["ddt"][bi, t, h] += float(x[bi, t, h] @ gB) + A[h] * q
                out["dA"][h] += dt[bi, t, h] * q
                out["dA_abs"][h] += abs(dt[bi, t, h] * q)
                out["dD"][h] += float(dy[bi, t, h] @ x[bi, t, h])
                g = abar * g                                            # dL/dh_{t-1}
            out["dinit"][s, h] = g
    return out

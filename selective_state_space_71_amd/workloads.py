"""Seeded synthetic inputs for the SSD layer.

This module only draws random numbers and rounds them to the input dtypes; it
holds none of the layer's arithmetic.  Both the GPU path (tests, bench) and
the fp64 CPU oracle consume exactly the arrays produced here, so bf16 inputs
are rounded once (round-to-nearest-even from fp32) and every consumer sees the
same values.

Workloads (shapes of the Mamba-2 layers discussed in "Transformers are SSMs
Review", section 3-2(4)-(6); no public dataset is involved):
  0 tiny_fp32     : b1 L256 H2 P16 N16 G1, chunk 64, fp32 io
  1 mamba2_130m   : b8 L2048 H24 P64 N128 G1, chunk 256, bf16 io
  2 mamba2_2p7b   : b4 L8192 H80 P64 N128 G1, chunk 256, bf16 io, init ~ N(0, 0.1)
  3 varlen_packed : 16 sequences, 65536 tokens, H32 P64 N128 G8, chunk 256, bf16
  4 decode        : b256 H80 P64 N128 G1, one token, state ~ N(0, 1)

Value recipe (all workloads): x ~ N(0,1); B, C ~ N(0,1)/sqrt(N);
dt = softplus(0.5 z + b_h) with z ~ N(0,1) and b_h = log(expm1(dt_h)), where
dt_h runs geometrically over the heads from 1e-3 to 1e-1; A_h = -exp(U(log 1,
log 16)); D_h ~ N(0,1).  Draw order: x, B, C, z, A, D, initial state,
sequence lengths.  Generator: numpy PCG64 seeded with 71000 + workload index.
"""
from __future__ import annotations

import math

import numpy as np

SEED_BASE = 71000

WORKLOADS = [
    dict(name="tiny_fp32", batch=1, seqlen=256, nheads=2, headdim=16, dstate=16,
         ngroups=1, chunk=64, io="f32", init_std=None),
    dict(name="mamba2_130m", batch=8, seqlen=2048, nheads=24, headdim=64, dstate=128,
         ngroups=1, chunk=256, io="bf16", init_std=None),
    dict(name="mamba2_2p7b", batch=4, seqlen=8192, nheads=80, headdim=64, dstate=128,
         ngroups=1, chunk=256, io="bf16", init_std=0.1),
    dict(name="varlen_packed", nseq=16, total=65536, lmin=64, lmax=8192, nheads=32,
         headdim=64, dstate=128, ngroups=8, chunk=256, io="bf16", init_std=None),
    dict(name="decode", batch=256, nheads=80, headdim=64, dstate=128, ngroups=1,
         io="bf16", state_std=1.0),
]


# --------------------------------------------------------------------------- bf16
def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the bits."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f64(a, io: str) -> np.ndarray:
    """Exact float64 view of an io-dtype array (bf16 given as uint16 bits)."""
    if io == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _round_io(a, io: str):
    a32 = np.asarray(a, dtype=np.float32)
    return f32_to_bf16_bits(a32) if io == "bf16" else np.ascontiguousarray(a32)


# --------------------------------------------------------------------------- pieces
def head_dt_targets(H: int) -> np.ndarray:
    """Per-head target step sizes, geometric from 1e-3 to 1e-1."""
    frac = np.arange(H, dtype=np.float64) / (H - 1) if H > 1 else np.array([0.5])
    return np.exp(math.log(1e-3) + frac * (math.log(1e-1) - math.log(1e-3)))


def softplus(v):
    return np.logaddexp(0.0, v)


def varlen_lengths(rng, nseq: int, total: int, lmin: int, lmax: int) -> np.ndarray:
    """Log-uniform lengths in [lmin, lmax] rescaled to sum to ``total``.

    Draw nseq log-uniform values; repeatedly rescale the unclipped ones to hit
    the target sum and clip to the bounds until nothing changes; then floor
    and hand the remainder (+1 each) to the largest fractional parts."""
    assert nseq * lmin <= total <= nseq * lmax
    v = np.exp(rng.uniform(math.log(lmin), math.log(lmax), size=nseq))
    for _ in range(200):
        clipped = (v <= lmin) | (v >= lmax)
        free = ~clipped
        rest = total - v[clipped].sum()
        if free.any() and v[free].sum() > 0:
            v[free] *= rest / v[free].sum()
        nv = np.clip(v, lmin, lmax)
        if np.allclose(nv, v) and abs(nv.sum() - total) < 1e-6 * total:
            v = nv
            break
        v = nv
    fl = np.floor(v).astype(np.int64)
    rem = int(total - fl.sum())
    order = np.argsort(-(v - fl), kind="stable")
    i = 0
    while rem > 0:
        j = order[i % nseq]
        if fl[j] < lmax:
            fl[j] += 1
            rem -= 1
        i += 1
    while rem < 0:
        j = order[::-1][i % nseq]
        if fl[j] > lmin:
            fl[j] -= 1
            rem += 1
        i += 1
    assert fl.sum() == total and fl.min() >= lmin and fl.max() <= lmax
    return fl


# --------------------------------------------------------------------------- public
def make_inputs(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int,
                ngroups: int = 1, io: str = "bf16", seed: int = 0,
                init_std=None, lengths=None):
    """Draw one forward-pass input set.

    Returns a dict with numpy arrays: x [b,L,H,P] and B, C [b,L,G,N] in the io
    dtype (bf16 as uint16 bits), dt [b,L,H], A [H], D [H], init_state
    [nseq,H,P,N] (or None) in float32, cu_seqlens (int32, or None) and the
    shape fields.  With ``lengths`` given, batch must be 1 and the tokens are
    packed back to back (seqlen == sum(lengths))."""
    rng = np.random.default_rng(seed)
    b, L, H, P, N, G = batch, seqlen, nheads, headdim, dstate, ngroups
    assert H % G == 0
    x = _round_io(rng.standard_normal((b, L, H, P), dtype=np.float32), io)
    scale = np.float32(1.0 / math.sqrt(N))
    Bm = _round_io(rng.standard_normal((b, L, G, N), dtype=np.float32) * scale, io)
    Cm = _round_io(rng.standard_normal((b, L, G, N), dtype=np.float32) * scale, io)
    z = rng.standard_normal((b, L, H))
    bias = np.log(np.expm1(head_dt_targets(H)))
    dt = softplus(0.5 * z + bias[None, None, :]).astype(np.float32)
    A = (-np.exp(rng.uniform(math.log(1.0), math.log(16.0), size=H))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    cu = None
    nseq = b
    if lengths is not None:
        assert b == 1 and int(np.sum(lengths)) == L
        cu = np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)
        nseq = len(lengths)
    init = None
    if init_std is not None:
        init = (rng.standard_normal((nseq, H, P, N), dtype=np.float32)
                * np.float32(init_std))
    return dict(x=x, dt=dt, A=A, B=Bm, C=Cm, D=D, init_state=init, cu_seqlens=cu,
                io=io, batch=b, seqlen=L, nheads=H, headdim=P, dstate=N, ngroups=G,
                nseq=nseq)


def make_decode_inputs(batch: int, nheads: int, headdim: int, dstate: int,
                       ngroups: int = 1, io: str = "bf16", seed: int = 0,
                       state_std: float = 1.0):
    """One decode step: state [b,H,P,N] f32, x [b,H,P], B/C [b,G,N] in io
    dtype, dt [b,H] f32 (same recipe as the forward), A, D [H] f32."""
    rng = np.random.default_rng(seed)
    b, H, P, N, G = batch, nheads, headdim, dstate, ngroups
    x = _round_io(rng.standard_normal((b, H, P), dtype=np.float32), io)
    scale = np.float32(1.0 / math.sqrt(N))
    Bm = _round_io(rng.standard_normal((b, G, N), dtype=np.float32) * scale, io)
    Cm = _round_io(rng.standard_normal((b, G, N), dtype=np.float32) * scale, io)
    z = rng.standard_normal((b, H))
    bias = np.log(np.expm1(head_dt_targets(H)))
    dt = softplus(0.5 * z + bias[None, :]).astype(np.float32)
    A = (-np.exp(rng.uniform(math.log(1.0), math.log(16.0), size=H))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    state = rng.standard_normal((b, H, P, N), dtype=np.float32) * np.float32(state_std)
    return dict(state=state, x=x, dt=dt, A=A, B=Bm, C=Cm, D=D, io=io, batch=b,
                nheads=H, headdim=P, dstate=N, ngroups=G)


def workload_inputs(index: int):
    """Inputs of one of the five named workloads (seed 71000 + index)."""
    w = WORKLOADS[index]
    seed = SEED_BASE + index
    if w["name"] == "decode":
        return make_decode_inputs(w["batch"], w["nheads"], w["headdim"], w["dstate"],
                                  w["ngroups"], w["io"], seed, w["state_std"])
    if w["name"] == "varlen_packed":
        # lengths are drawn last, from a generator of their own seeded the
        # same way, so the token count (and thus the other arrays' shapes)
        # is known before the lengths are drawn.
        lens = varlen_lengths(np.random.default_rng([seed, 1]), w["nseq"], w["total"],
                              w["lmin"], w["lmax"])
        return make_inputs(1, w["total"], w["nheads"], w["headdim"], w["dstate"],
                           w["ngroups"], w["io"], seed, w["init_std"], lengths=lens)
    return make_inputs(w["batch"], w["seqlen"], w["nheads"], w["headdim"], w["dstate"],
                       w["ngroups"], w["io"], seed, w["init_std"])


def make_block_inputs(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int,
                      ngroups: int = 1, width: int = 4, io: str = "bf16", seed: int = 0,
                      lengths=None, with_state: bool = True):
    """Draw inputs for the block prologue and epilogue.

    Prologue: xbc [b, L, H*P + 2*G*N] in the io dtype (the fused projection
    output, N(0, 1)), conv weight [channels, width] and bias [channels] in
    float32 drawn U(-1/sqrt(width), 1/sqrt(width)) (the default initialisation
    of a depthwise convolution with `width` inputs per output), conv_state
    [nseq, width-1, channels] in the io dtype (N(0, 1)) or None.
    Epilogue: y and z [b, L, H*P] in the io dtype (N(0, 1)) and the norm weight
    [H*P] float32 ~ 1 + N(0, 0.1^2).  With ``lengths`` the batch is 1 and the
    sequences are packed (cu_seqlens)."""
    rng = np.random.default_rng(seed)
    b, L = batch, seqlen
    HP, GN = nheads * headdim, ngroups * dstate
    Cc = HP + 2 * GN
    bound = np.float32(1.0 / math.sqrt(width))
    cu = None
    nseq = b
    if lengths is not None:
        assert b == 1 and int(np.sum(lengths)) == L
        cu = np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)
        nseq = len(lengths)
    return dict(
        xbc=_round_io(rng.standard_normal((b, L, Cc), dtype=np.float32), io),
        conv_w=rng.uniform(-bound, bound, size=(Cc, width)).astype(np.float32),
        conv_b=rng.uniform(-bound, bound, size=Cc).astype(np.float32),
        conv_state=(_round_io(rng.standard_normal((nseq, width - 1, Cc), dtype=np.float32), io)
                    if with_state else None),
        y=_round_io(rng.standard_normal((b, L, HP), dtype=np.float32), io),
        z=_round_io(rng.standard_normal((b, L, HP), dtype=np.float32), io),
        norm_w=(1.0 + 0.1 * rng.standard_normal(HP)).astype(np.float32),
        cu_seqlens=cu, io=io, batch=b, seqlen=L, nheads=nheads, headdim=headdim, dstate=dstate,
        ngroups=ngroups, width=width, nseq=nseq)

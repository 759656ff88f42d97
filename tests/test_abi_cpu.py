"""CPU-only checks of the C ABI: the library loads, exports every function
include/ssd.h declares, and rejects invalid calls synchronously (every case
here fails validation before anything could be launched)."""
import ctypes
import os
import subprocess

import pytest

from selective_state_space_71_amd import ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssd.LIB_PATH):
        from selective_state_space_71_amd import build
        build.build(verbose=False)
    return ssd.load_library()


def test_header_symbols_are_exported(lib):
    names = ssd.header_functions()
    assert {"ssd_chunk_scan_fwd", "ssd_decode_step", "ssd_chunk_scan_fwd_workspace_size",
            "ssd_status_string", "ssd_abi_version", "ssd_chunk_scan_fwd_check",
            "ssd_chunk_scan_fwd_ex", "ssd_decode_step_ex", "ssd_causal_conv1d_fwd",
            "ssd_gated_rmsnorm_fwd", "ssd_chunk_scan_bwd", "ssd_chunk_scan_bwd_workspace_size",
            "ssd_chunk_scan_fwd_noalloc"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", ssd.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_abi_version_and_status_strings(lib):
    assert lib.ssd_abi_version() == 5
    for code, name in ssd._STATUS.items():
        assert lib.ssd_status_string(code).decode().startswith(name)
    assert b"unknown" in lib.ssd_status_string(77)


def _dims(**kw):
    d = dict(batch=2, seqlen=512, nheads=8, headdim=64, dstate=128, ngroups=1, nseq=2)
    d.update(kw)
    return ssd.SsdDims(*[d[k] for k in ("batch", "seqlen", "nheads", "headdim", "dstate",
                                         "ngroups", "nseq")])


FAKE = 1 << 40   # never dereferenced: every call below fails validation first


def _fwd(lib, dims, io=ssd.SSD_BF16, Q=256, **ptrs):
    dp = dict(x=FAKE, dt=FAKE + (1 << 30), A=FAKE + (2 << 30), B=FAKE + (3 << 30),
              C=FAKE + (4 << 30), D=None, init=None, cu=None, y=FAKE + (8 << 30), fin=None,
              ws=FAKE + (16 << 30), wsb=1 << 40)
    dp.update(ptrs)
    return lib.ssd_chunk_scan_fwd(
        ctypes.byref(dims) if dims is not None else None, io, Q, dp["x"], dp["dt"], dp["A"],
        dp["B"], dp["C"], dp["D"], dp["init"], dp["cu"], dp["y"], dp["fin"], dp["ws"],
        ctypes.c_size_t(dp["wsb"]), None)


def test_workspace_size_query(lib):
    n = lib.ssd_chunk_scan_fwd_workspace_size(ctypes.byref(_dims()), 256, ssd.SSD_BF16)
    assert n >= 2 * 8 * 64 * 128 * 4            # holds the fp32 boundary states
    assert n % 256 == 0
    assert lib.ssd_chunk_scan_fwd_workspace_size(ctypes.byref(_dims()), 100, ssd.SSD_BF16) == 0
    assert lib.ssd_chunk_scan_fwd_workspace_size(None, 256, ssd.SSD_BF16) == 0
    assert lib.ssd_chunk_scan_fwd_workspace_size(ctypes.byref(_dims(headdim=48)), 256, ssd.SSD_BF16) == 0
    assert lib.ssd_chunk_scan_fwd_workspace_size(ctypes.byref(_dims()), 128, ssd.SSD_F32) > 0
    assert lib.ssd_chunk_scan_fwd_workspace_size(ctypes.byref(_dims(headdim=16, dstate=16)), 64, ssd.SSD_F32) > 0
    # every head dim in {16, 32, 64, 128}, state dim in {16, ..., 256} and chunk
    # length in {64, 128, 256} is accepted in both dtypes (a chunk whose tiles
    # exceed LDS runs as the largest shorter chunk that fits; a shorter chunk
    # needs a larger schedule, never a smaller one)
    for io in (ssd.SSD_BF16, ssd.SSD_F32):
        for P in (16, 32, 64, 128):
            for N in (16, 32, 64, 128, 256):
                sizes = [lib.ssd_chunk_scan_fwd_workspace_size(ctypes.byref(_dims(headdim=P, dstate=N)), Q, io)
                         for Q in (64, 128, 256)]
                assert min(sizes) > 0, (io, P, N, sizes)
                assert sizes[0] >= sizes[1] >= sizes[2], (io, P, N, sizes)


@pytest.mark.parametrize("case,expect", [
    (dict(dims=None), 1),
    (dict(io=5), 3),
    (dict(dims=_dims(seqlen=0)), 2),
    (dict(dims=_dims(nheads=6, ngroups=4)), 2),
    (dict(dims=_dims(nseq=3)), 2),                               # dense needs nseq == batch
    (dict(Q=100), 4),
    (dict(dims=_dims(headdim=48)), 4),
    (dict(dims=_dims(dstate=48)), 4),                            # state dim not built
    (dict(dims=_dims(headdim=256)), 4),                          # head dim not built
    (dict(dims=_dims(nheads=1 << 14, ngroups=1)), 2),            # one chunk of x would span 2^30 bytes
    (dict(x=None), 1),
    (dict(A=None), 1),
    (dict(ws=None), 7),
    (dict(x=FAKE + 2), 5),
    (dict(ws=FAKE + (16 << 30) + 16), 5),
    (dict(y=FAKE + 64), 6),                                      # y overlaps x
    (dict(fin=FAKE + (3 << 30)), 6),                             # final_state overlaps B
    (dict(wsb=1024), 7),
])
def test_forward_validation_rejects(lib, case, expect):
    dims = case.pop("dims", _dims())
    assert _fwd(lib, dims, **case) == expect


def test_varlen_validation(lib):
    # cu_seqlens needs batch == 1
    assert _fwd(lib, _dims(), cu=FAKE + (20 << 30)) == 2
    # and nseq <= 65536
    assert _fwd(lib, _dims(batch=1, nseq=70000), cu=FAKE + (20 << 30)) == 2
    # a packed batch of a size that is not built is reported as unsupported,
    # not as a layout error (the binding relies on this to name the reason)
    assert _fwd(lib, _dims(batch=1, nseq=5, headdim=48, dstate=128), io=ssd.SSD_F32,
                cu=FAKE + (20 << 30)) == 4


def _dec(lib, dims, io=ssd.SSD_BF16, **ptrs):
    dp = dict(state=FAKE, x=FAKE + (1 << 34), dt=FAKE + (2 << 34), A=FAKE + (3 << 34),
              B=FAKE + (4 << 34), C=FAKE + (5 << 34), D=None, y=FAKE + (6 << 34))
    dp.update(ptrs)
    return lib.ssd_decode_step(ctypes.byref(dims) if dims is not None else None, io, dp["state"],
                               dp["x"], dp["dt"], dp["A"], dp["B"], dp["C"], dp["D"], dp["y"], None)


@pytest.mark.parametrize("case,expect", [
    (dict(dims=None), 1),
    (dict(io=9), 3),
    (dict(dims=_dims(nheads=0)), 2),
    (dict(dims=_dims(dstate=48)), 4),
    (dict(state=None), 1),
    (dict(y=None), 1),
    (dict(x=FAKE + (1 << 34) + 8), 5),
    (dict(y=FAKE + 16), 6),                                      # y overlaps state
    (dict(x=FAKE + 32), 6),                                      # x overlaps state
])
def test_decode_validation_rejects(lib, case, expect):
    dims = case.pop("dims", _dims())
    assert _dec(lib, dims, **case) == expect


def _opts(bias=None, softplus=1, lo=-float("inf"), hi=float("inf")):
    return ssd.SsdDtOpts(bias, softplus, lo, hi)


@pytest.mark.parametrize("opts,expect", [
    (_opts(lo=1.0, hi=0.5), 2),                                  # dt_min > dt_max
    (_opts(lo=float("nan")), 2),                                 # NaN bound
    (_opts(bias=FAKE + (1 << 30) + 4), 5),                       # misaligned dt_bias
    (_opts(bias=FAKE + (8 << 30) + 64), 6),                      # dt_bias overlaps y
])
def test_dt_options_validation(lib, opts, expect):
    # forward: same fake pointers as _fwd, through the _ex entry point
    dims = _dims()
    rc = lib.ssd_chunk_scan_fwd_ex(ctypes.byref(dims), ssd.SSD_BF16, 256, ctypes.byref(opts), FAKE,
                                   FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30), FAKE + (4 << 30),
                                   None, None, None, FAKE + (8 << 30), None, FAKE + (16 << 30),
                                   ctypes.c_size_t(1 << 40), None)
    assert rc == expect
    if expect == 6:
        opts = _opts(bias=FAKE + (6 << 34) + 64)                 # overlaps the decode y
    rc = lib.ssd_decode_step_ex(ctypes.byref(dims), ssd.SSD_BF16, ctypes.byref(opts), FAKE,
                                FAKE + (1 << 34), FAKE + (2 << 34), FAKE + (3 << 34), FAKE + (4 << 34),
                                FAKE + (5 << 34), None, FAKE + (6 << 34), None)
    assert rc == expect


def _conv(lib, dims, io=ssd.SSD_BF16, width=4, **ptrs):
    dp = dict(xbc=FAKE, w=FAKE + (1 << 34), b=None, st=None, cu=None, x=FAKE + (2 << 34), B=FAKE + (3 << 34),
              C=FAKE + (4 << 34), so=None)
    dp.update(ptrs)
    return lib.ssd_causal_conv1d_fwd(ctypes.byref(dims) if dims is not None else None, io, width, dp["xbc"],
                                     dp["w"], dp["b"], 1, dp["st"], dp["cu"], dp["x"], dp["B"], dp["C"],
                                     dp["so"], None)


@pytest.mark.parametrize("case,expect", [
    (dict(dims=None), 1),
    (dict(io=4), 3),
    (dict(width=0), 4),
    (dict(width=5), 4),
    (dict(dims=_dims(headdim=12)), 4),
    (dict(dims=_dims(dstate=20)), 4),
    (dict(dims=_dims(nseq=3)), 2),                               # dense needs nseq == batch
    (dict(cu=FAKE + (5 << 34)), 2),                              # varlen needs batch == 1
    (dict(x=None), 1),
    (dict(w=None), 1),
    (dict(B=FAKE + (3 << 34) + 8), 5),
    (dict(x=FAKE + 64), 6),                                      # x overlaps xbc
    (dict(C=FAKE + (3 << 34) + 64), 6),                          # C overlaps B
    (dict(st=FAKE + (6 << 34), so=FAKE + (6 << 34)), 6),         # state out over state in
])
def test_conv_validation_rejects(lib, case, expect):
    dims = case.pop("dims", _dims())
    assert _conv(lib, dims, **case) == expect


def _norm(lib, rows=16, dim=5120, gs=5120, io=ssd.SSD_BF16, eps=1e-5, **ptrs):
    dp = dict(y=FAKE, z=FAKE + (1 << 34), w=FAKE + (2 << 34), out=FAKE + (3 << 34))
    dp.update(ptrs)
    return lib.ssd_gated_rmsnorm_fwd(rows, dim, gs, io, dp["y"], dp["z"], dp["w"], ctypes.c_float(eps), 0,
                                     dp["out"], None)


@pytest.mark.parametrize("case,expect", [
    (dict(io=2), 3),
    (dict(rows=0), 2),
    (dict(gs=1000), 2),                                          # does not divide dim
    (dict(dim=60, gs=12), 4),                                    # not a multiple of 8
    (dict(dim=16384, gs=16384), 4),                              # bf16 groups up to 8192
    (dict(dim=8192, gs=8192, io=ssd.SSD_F32), 4),                # fp32 groups up to 4096
    (dict(eps=-1.0), 2),
    (dict(eps=float("nan")), 2),
    (dict(y=None), 1),
    (dict(w=None), 1),
    (dict(out=FAKE + (3 << 34) + 4), 5),
    (dict(out=FAKE + 64), 6),                                    # partial overlap with y
    (dict(out=FAKE + (2 << 34)), 6),                             # over the weight
])
def test_norm_validation_rejects(lib, case, expect):
    assert _norm(lib, **case) == expect



def _bwd(lib, dims, io=ssd.SSD_BF16, **ptrs):
    base = FAKE
    names = ["x", "dt", "A", "B", "C", "D", "init", "cu", "dy", "dfin", "dx", "ddt", "dA", "dB", "dC", "dD",
             "dinit"]
    dp = {n: base + ((i + 1) << 34) for i, n in enumerate(names)}
    for n in ("D", "init", "cu", "dfin", "dinit"):
        dp[n] = None
    dp.update(ws=FAKE + (40 << 34), wsb=1 << 40)
    dp.update(ptrs)
    return lib.ssd_chunk_scan_bwd(ctypes.byref(dims) if dims is not None else None, io,
                                  *[dp[n] for n in names], dp["ws"], ctypes.c_size_t(dp["wsb"]), None)


def test_bwd_workspace_size_query(lib):
    n = lib.ssd_chunk_scan_bwd_workspace_size(ctypes.byref(_dims()), ssd.SSD_BF16)
    # every boundary state and state gradient of 512/64 chunks x 2 sequences x 8 heads
    assert n >= 2 * 2 * 8 * 8 * 64 * 128 * 4 and n % 256 == 0
    # head dim 128 runs as two kernel heads of 64 (their dA, dD partials are
    # kept apart until the reduction)
    n128 = lib.ssd_chunk_scan_bwd_workspace_size(ctypes.byref(_dims(headdim=128)), ssd.SSD_BF16)
    assert n128 >= 2 * 2 * 8 * 8 * 128 * 128 * 4 and n128 % 256 == 0
    assert lib.ssd_chunk_scan_bwd_workspace_size(ctypes.byref(_dims(headdim=128, dstate=64)), ssd.SSD_F32) > 0
    assert lib.ssd_chunk_scan_bwd_workspace_size(ctypes.byref(_dims(headdim=48)), ssd.SSD_BF16) == 0
    assert lib.ssd_chunk_scan_bwd_workspace_size(ctypes.byref(_dims(dstate=48)), ssd.SSD_BF16) == 0
    # state dims beyond the kernels' (bf16 256, fp32 128 and 256) run in slices
    # of the state dim: the workspace also holds the slices' inputs and terms
    n64 = lib.ssd_chunk_scan_bwd_workspace_size(ctypes.byref(_dims(dstate=64)), ssd.SSD_F32)
    n128 = lib.ssd_chunk_scan_bwd_workspace_size(ctypes.byref(_dims(dstate=128)), ssd.SSD_F32)
    assert n64 > 0 and n128 > n64
    for io, N in ((ssd.SSD_BF16, 256), (ssd.SSD_F32, 256)):
        assert lib.ssd_chunk_scan_bwd_workspace_size(ctypes.byref(_dims(dstate=N)), io) > 0
    # the scans address a 64-token chunk of x, dy, B or C rows with 32-bit
    # byte offsets: 2^22 channels of fp32-sized rows reach 2^30 bytes
    assert lib.ssd_chunk_scan_bwd_workspace_size(ctypes.byref(_dims(nheads=65536 - 1)), ssd.SSD_BF16) > 0
    assert lib.ssd_chunk_scan_bwd_workspace_size(ctypes.byref(_dims(nheads=65536)), ssd.SSD_BF16) == 0


@pytest.mark.parametrize("case,expect", [
    (dict(dims=None), 1),
    (dict(io=7), 3),
    (dict(dims=_dims(headdim=48)), 4),
    (dict(dims=_dims(dstate=48)), 4),
    (dict(dims=_dims(nseq=3)), 2),
    (dict(dy=None), 1),
    (dict(dB=None), 1),
    (dict(ws=None), 7),
    (dict(wsb=4096), 7),
    (dict(dx=FAKE + (11 << 34) + 8), 5),
    (dict(dx=FAKE + (9 << 34)), 6),                              # dx over dy
    (dict(dC=FAKE + (14 << 34) + 64), 6),                        # dC over dB
    (dict(ddt=FAKE + (40 << 34) + 256), 6),                      # ddt inside the workspace
])
def test_bwd_validation_rejects(lib, case, expect):
    dims = case.pop("dims", _dims())
    assert _bwd(lib, dims, **case) == expect


def _fwd_noalloc(lib, dims, io=ssd.SSD_BF16, Q=256, **ptrs):
    dp = dict(x=FAKE, dt=FAKE + (1 << 30), A=FAKE + (2 << 30), B=FAKE + (3 << 30),
              C=FAKE + (4 << 30), D=None, init=None, cu=None, y=FAKE + (8 << 30), fin=None)
    dp.update(ptrs)
    return lib.ssd_chunk_scan_fwd_noalloc(
        ctypes.byref(dims) if dims is not None else None, io, Q, None, dp["x"], dp["dt"], dp["A"],
        dp["B"], dp["C"], dp["D"], dp["init"], dp["cu"], dp["y"], dp["fin"], None)


@pytest.mark.parametrize("case,expect", [
    (dict(dims=None), 1),
    (dict(io=5), 3),
    (dict(Q=100), 4),
    (dict(dims=_dims(headdim=48)), 4),
    (dict(x=None), 1),
    (dict(x=FAKE + 2), 5),
    (dict(y=FAKE + 64), 6),
    # 16 sequences x 80 heads of 64 x 128 fp32 boundary states (42 MB) do not
    # fit the 32 MiB scratch when final_state is NULL
    (dict(dims=_dims(batch=16, nseq=16, seqlen=1024, nheads=80)), 7),
])
def test_noalloc_forward_validation_rejects(lib, case, expect):
    """The allocation-free forward validates like the workspace one and
    rejects schedules beyond its scratch array before touching the device."""
    dims = case.pop("dims", _dims())
    assert _fwd_noalloc(lib, dims, **case) == expect


# (last: it reloads the binding module, which redefines its ctypes structures)
def test_binding_fails_loudly_without_library(tmp_path):
    import importlib
    mod = importlib.reload(ssd)
    try:
        mod._lib = None
        with pytest.raises(RuntimeError, match="not built"):
            mod.load_library(str(tmp_path / "missing.so"))
    finally:
        importlib.reload(ssd)


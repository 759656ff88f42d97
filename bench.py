"""Benchmark of the SSD forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one ssd_chunk_scan_fwd call over one batch of the Mamba-2 2.7B layer
shape (batch 4, L 8192, 80 heads x 64, state 128, 1 group, chunk 256, bf16
x/B/C, fp32 dt/A/D/state, random fp32 initial state).  Inputs are seeded
synthetic data resident in HBM before timing starts.  Prints one JSON line.

The roofline object reports the fused forward kernel against HBM bandwidth
(its algorithmic bytes are the compulsory traffic; see the design doc for the
per-token figures) and, in "mfma", its algorithmic bf16 MFMA rate.  The
"cpu_baseline" is the fp64 oracle timed on this host's cores over the whole
workload.  The 130M-layer shape and the packed
variable-length batch are reported under "workloads" (parity configurations;
the headline line is the 2.7B layer).  A decode line for the b256 H80 P64 N128
single-token step is included under "decode", and the block prologue (causal convolution of the
fused x|B|C projection) and epilogue (gated RMSNorm) at the same 2.7B layer
shape under "block" (skip with --no-block), and the backward pass
(ssd_chunk_scan_bwd, all gradients) at the forward's workload under
"backward" (skip with --no-bwd).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FWD_INDEX = 2                  # Mamba-2 2.7B layer shape
DEC_INDEX = 4                  # decode, b256


def fwd_algorithmic(w, lengths=None, init_state=True):
    """Algorithmic bytes and MFMA flops of one forward pass.

    Bytes: the compulsory HBM traffic -- read x, dt, B, C (and the initial
    state when there is one), write y and the final state (A, D negligible).
    Flops, per chunk of q tokens (the last chunk of a sequence may be
    partial): per head, the causal half of the diagonal block q (q+1) P, and
    per token the chunk-state formation 2 N P and the state read-out 2 N P;
    per group, the causal half of C B^T, q (q+1) N.  ``lengths`` lists the
    sequence lengths of a packed batch (default: batch x seqlen)."""
    H, P, N, G, Q = w["nheads"], w["headdim"], w["dstate"], w["ngroups"], w["chunk"]
    if lengths is None:
        lengths = [w["seqlen"]] * w["batch"]
    tok = int(sum(lengths))
    nseq = len(lengths)
    io = 2
    byts = tok * (H * P * io * 2 + H * 4 + G * N * io * 2) + (2 if init_state else 1) * nseq * H * P * N * 4
    pairs = 0
    for L in lengths:
        full, rest = divmod(int(L), Q)
        pairs += full * Q * (Q + 1) // 2 + rest * (rest + 1) // 2
    flops = 2 * pairs * (H * P + G * N) + tok * H * 4 * N * P
    return float(byts), float(flops)


def dec_algorithmic(w):
    b, H, P, N, G = w["batch"], w["nheads"], w["headdim"], w["dstate"], w["ngroups"]
    return float(8 * b * H * P * N + b * H * P * 2 * 2 + b * H * 4 + 2 * b * G * N * 2)


def time_calls(fn, stream, nrep=30):
    """Average µs of fn() over nrep calls, HIP events on `stream`."""
    import torch
    for _ in range(3):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(nrep):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / nrep * 1e3


def bench_block(w, stream, to_dev):
    """Prologue and epilogue at the forward workload's shape (bf16 io).

    Algorithmic bytes: the convolution reads the fused projection and writes
    x, B and C once (2 * tokens * channels * 2 bytes; weights negligible); the
    gated RMSNorm reads y and z and writes its output (3 * tokens * H*P * 2)."""
    import torch
    from selective_state_space_71_amd import ssd, workloads as wl
    b, L, H, P, N, G = w["batch"], w["seqlen"], w["nheads"], w["headdim"], w["dstate"], w["ngroups"]
    d = wl.make_block_inputs(b, L, H, P, N, G, 4, "bf16", seed=7100, with_state=False)
    tok = b * L
    res = {"workload": f"batch {b}, L {L}, {H * P} + 2*{G * N} channels, conv width 4, SiLU; "
                       f"gated RMSNorm over {H * P} channels, one group, bf16"}
    xbc = to_dev(d["xbc"], True)
    cw, cb = to_dev(d["conv_w"], False), to_dev(d["conv_b"], False)
    x = torch.empty((b, L, H, P), dtype=torch.bfloat16, device="cuda")
    Bo = torch.empty((b, L, G, N), dtype=torch.bfloat16, device="cuda")
    Co = torch.empty_like(Bo)
    us = time_calls(lambda: ssd.causal_conv1d_fwd(xbc, cw, H, P, G, N, bias=cb, x=x, B=Bo, C=Co), stream)
    byts = 2.0 * tok * (H * P + 2 * G * N) * 2
    res["conv"] = {"us": us, "alg_bytes": byts, "achieved_gbs": byts / (us * 1e-6) / 1e9,
                   "peak_gbs": HBM_PEAK_GBS, "frac": byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    del xbc, x, Bo, Co
    y, z = to_dev(d["y"], True), to_dev(d["z"], True)
    nw = to_dev(d["norm_w"], False)
    o = torch.empty_like(y)
    us = time_calls(lambda: ssd.gated_rmsnorm_fwd(y, z, nw, eps=1e-5, out=o), stream)
    byts = 3.0 * tok * H * P * 2
    res["gated_rmsnorm"] = {"us": us, "alg_bytes": byts, "achieved_gbs": byts / (us * 1e-6) / 1e9,
                            "peak_gbs": HBM_PEAK_GBS, "frac": byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    return res


def bwd_algorithmic(w, Qb=64):
    """Algorithmic bytes and MFMA flops of one backward pass.

    Bytes: read x, dy, dt, B, C, the initial state and the final-state
    gradient; write dx, ddt, dB and dC (fp32) and the initial-state gradient.
    Flops per (token, head), with the backward's 64-token chunks: the causal
    halves of dY X^T, M^T dY, W^T C and W B, 2 Q (P + N); the low-rank terms
    B R^T, X R and dY H, 6 P N; the two chunk-state contractions of the scans,
    4 P N.  Per (token, group): the causal half of C B^T, Q N."""
    b, L, H, P, N, G = w["batch"], w["seqlen"], w["nheads"], w["headdim"], w["dstate"], w["ngroups"]
    tok = b * L
    byts = tok * (H * P * 2 * 3 + H * 4 * 2 + G * N * (2 * 2 + 4 * 2)) + 3 * b * H * P * N * 4
    flops = tok * H * (2 * Qb * (P + N) + 10 * P * N) + tok * G * Qb * N
    return float(byts), float(flops)


def bench_backward(w, stream, x, dt, A, B, C, D, h0):
    import torch
    from selective_state_space_71_amd import ssd
    g = torch.Generator(device=x.device)
    g.manual_seed(7101)
    dy = torch.randn(x.shape, generator=g, device=x.device).to(torch.bfloat16)
    dfin = torch.randn(h0.shape, generator=g, device=x.device)
    ssd.chunk_scan_bwd(x, dt, A, B, C, dy, D=D, init_state=h0, dfinal_state=dfin)
    ws = ssd.chunk_scan_bwd.last_workspace
    us = time_calls(lambda: ssd.chunk_scan_bwd(x, dt, A, B, C, dy, D=D, init_state=h0, dfinal_state=dfin,
                                               workspace=ws), stream, nrep=10)
    byts, flops = bwd_algorithmic(w)
    tok = w["batch"] * w["seqlen"]
    res = {"workload": "backward of the forward workload above: all gradients (dx bf16; ddt, dA, dB, dC, dD, "
                       "dinit fp32), 64-token chunks",
           "us": us, "tokens_per_s": tok / (us * 1e-6),
           "alg_bytes": byts, "achieved_gbs": byts / (us * 1e-6) / 1e9, "hbm_frac": byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
           "alg_flops": flops, "achieved_tflops": flops / (us * 1e-6) / 1e12,
           "mfma_frac": flops / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS,
           "workspace_bytes": int(ws.numel())}
    del ws
    return res


def bench_other_forward(stream, to_dev):
    """The Mamba-2 130M layer shape and the packed variable-length batch:
    time per call (HIP events over 20 calls on the launch stream), tokens/s,
    and the algorithmic HBM and MFMA rates against the MI355X peaks."""
    import torch
    from selective_state_space_71_amd import ssd, workloads as wl
    res = {}
    for idx, label in ((1, "mamba2_130m_layer: batch 8, L 2048, H 24, P 64, N 128, G 1, chunk 256, bf16"),
                       (3, "varlen_packed: 16 sequences, 65,536 tokens, H 32, P 64, N 128, G 8, chunk 256, bf16")):
        w = wl.WORKLOADS[idx]
        inp = wl.workload_inputs(idx)
        x, B, C = (to_dev(inp[k], True) for k in ("x", "B", "C"))
        dt, A, D = (to_dev(inp[k], False) for k in ("dt", "A", "D"))
        h0 = to_dev(inp["init_state"], False) if inp.get("init_state") is not None else None
        cu_np = inp.get("cu_seqlens")
        cu = torch.from_numpy(cu_np.astype(np.int32)).to(x.device) if cu_np is not None else None
        ssd.chunk_scan_fwd(x, dt, A, B, C, D, chunk_len=w["chunk"], init_state=h0, cu_seqlens=cu, check=True)
        ws = ssd.chunk_scan_fwd.last_workspace
        y = torch.empty_like(x)
        us = time_calls(lambda: ssd.chunk_scan_fwd(x, dt, A, B, C, D, chunk_len=w["chunk"], init_state=h0,
                                                   cu_seqlens=cu, y=y, workspace=ws), stream, nrep=20)
        assert ssd.check_workspace(ws) == 0
        lengths = None if cu_np is None else [int(cu_np[i + 1] - cu_np[i]) for i in range(len(cu_np) - 1)]
        wv = dict(w, seqlen=w.get("seqlen", 0), batch=w.get("batch", 1))
        byts, flops = fwd_algorithmic(wv, lengths=lengths, init_state=h0 is not None)
        tok = x.shape[0] * x.shape[1]
        gbs = byts / (us * 1e-6) / 1e9
        tfl = flops / (us * 1e-6) / 1e12
        res[w["name"]] = {"workload": label, "us": us, "tokens_per_s": tok / (us * 1e-6),
                          "alg_bytes": byts, "achieved_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                          "alg_flops": flops, "achieved_tflops": tfl, "mfma_frac": tfl / BF16_PEAK_TFLOPS}
        del x, B, C, dt, A, D, h0, cu, ws, y
    return res


def profile_forward(idx, warmup, steps, dev):
    """Forward calls of one workload only (for a profiler run): W untimed
    calls, then K calls, then a device-failure check."""
    import torch
    from selective_state_space_71_amd import ssd, workloads as wl
    w = wl.WORKLOADS[idx]
    inp = wl.workload_inputs(idx)

    def to_dev(a, bf16):
        if bf16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    io = inp["io"] == "bf16"
    x, B, C = (to_dev(inp[k], io) for k in ("x", "B", "C"))
    dt, A, D = (to_dev(inp[k], False) for k in ("dt", "A", "D"))
    h0 = to_dev(inp["init_state"], False) if inp.get("init_state") is not None else None
    cu = inp.get("cu_seqlens")
    cu = torch.from_numpy(cu.astype(np.int32)).to(dev) if cu is not None else None
    y = torch.empty_like(x)
    ssd.chunk_scan_fwd(x, dt, A, B, C, D, chunk_len=w["chunk"], init_state=h0, cu_seqlens=cu, y=y)
    ws = ssd.chunk_scan_fwd.last_workspace
    for _ in range(warmup + steps):
        ssd.chunk_scan_fwd(x, dt, A, B, C, D, chunk_len=w["chunk"], init_state=h0, cu_seqlens=cu, y=y,
                           workspace=ws)
    torch.cuda.synchronize()
    assert ssd.check_workspace(ws) == 0
    print(f"[bench] profiled {warmup + steps + 1} forward calls of workload {w['name']}", file=sys.stderr)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def kernel_source_sha():
    h = hashlib.sha256()
    for f in ("ssd_fwd_kernel.h", "ssd_device.h", "ssd_fwd_launch.h"):
        with open(os.path.join(ROOT, "selective_state_space_71_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per launch measured with rocprofv3 counters (profiles/), or
    None when absent or taken from a different kernel source."""
    path = os.path.join(ROOT, "profiles", "fwd_traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha") != kernel_source_sha():
        return None
    return rec.get("traffic_bytes")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-block", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--profile-workload", type=int, default=None, metavar="W",
                    help="profiling aid: run only W warm-up plus --steps forward calls of workload W "
                         "(1: 130M layer, 2: 2.7B layer, 3: packed batch) and print nothing else")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device copy (reference kernel for scaling "
                         "the FETCH_SIZE / WRITE_SIZE counters of a profiler run)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the SSD forward shards by (sequence, head) "
              "with no exchange, so N GPUs run N independent copies; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from selective_state_space_71_amd import ssd
    from selective_state_space_71_amd import workloads as wl

    ssd.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.profile_workload is not None:
        profile_forward(args.profile_workload, args.warmup, args.steps, dev)
        return
    w = wl.WORKLOADS[FWD_INDEX]
    inp = wl.workload_inputs(FWD_INDEX)

    def to_dev(a, bf16):
        if bf16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    x, B, C = (to_dev(inp[k], True) for k in ("x", "B", "C"))
    dt, A, D, h0 = (to_dev(inp[k], False) for k in ("dt", "A", "D", "init_state"))
    y = torch.empty_like(x)
    fin = torch.empty_like(h0)
    y, fin = ssd.chunk_scan_fwd(x, dt, A, B, C, D, chunk_len=w["chunk"], init_state=h0, y=y,
                                final_state=fin)
    ws = ssd.chunk_scan_fwd.last_workspace
    stream = torch.cuda.current_stream(dev)

    def step():
        ssd.chunk_scan_fwd(x, dt, A, B, C, D, chunk_len=w["chunk"], init_state=h0, y=y,
                           final_state=fin, workspace=ws)

    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert ssd.check_workspace(ws) == 0
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for k in range(args.steps):
        step()
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps)]
    ms_total = ev[0].elapsed_time(ev[-1])
    ms_step = ms_total / args.steps
    assert ssd.check_workspace(ws) == 0
    tokens = w["batch"] * w["seqlen"]
    byts, flops = fwd_algorithmic(w)
    ms_launch = float(np.mean(per))
    gbs = byts / (ms_launch * 1e-3) / 1e9
    tfl = flops / (ms_launch * 1e-3) / 1e12
    print(f"[bench] fwd {ms_step * 1e3:.1f} us/step (median {np.median(per) * 1e3:.1f}), "
          f"{gbs:.0f} GB/s alg, {tfl:.1f} TFLOP/s alg", file=sys.stderr, flush=True)
    out = {
        "metric": "SSD fwd tokens/s at Mamba-2 2.7B layer shape, L=8192; % bf16 MFMA peak",
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mamba2_2p7b_layer: batch 4, L 8192, H 80, P 64, N 128, G 1, "
                               "chunk 256, bf16 x/B/C, fp32 dt/A/D/state, init state N(0,0.1)",
                   "global_batch": w["batch"], "seq_len": w["seqlen"], "parallelism": "single_gpu"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": load_traffic(),
                     "kernel": "ssd_fwd_kernel (plus the tiny schedule kernel in the same launch)",
                     "alg_bytes_per_launch": byts, "launch_us": ms_launch * 1e3},
        "mfma": {"achieved": tfl, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": tfl / BF16_PEAK_TFLOPS, "alg_flops_per_launch": flops},
        "wall_s_timed": wall,
    }

    out["workloads"] = bench_other_forward(stream, to_dev)

    if not args.no_decode:
        wd = wl.WORKLOADS[DEC_INDEX]
        di = wl.workload_inputs(DEC_INDEX)
        st = to_dev(di["state"], False)
        dx, dB, dC = (to_dev(di[k], True) for k in ("x", "B", "C"))
        ddt, dA, dD = (to_dev(di[k], False) for k in ("dt", "A", "D"))
        dy = torch.empty_like(dx)
        for _ in range(3):
            ssd.decode_step(st, dx, ddt, dA, dB, dC, dD, y=dy)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nrep = 50
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(nrep):
            ssd.decode_step(st, dx, ddt, dA, dB, dC, dD, y=dy)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / nrep * 1e3
        db = dec_algorithmic(wd)
        out["decode"] = {"workload": "decode: batch 256, H 80, P 64, N 128, G 1, fp32 state",
                         "tokens_per_s": wd["batch"] / (us * 1e-6), "us_per_step": us,
                         "achieved_gbs": db / (us * 1e-6) / 1e9, "peak_gbs": HBM_PEAK_GBS,
                         "frac": db / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
        del st, dx, dB, dC, ddt, dA, dD, dy

    if not args.no_block:
        out["block"] = bench_block(w, stream, to_dev)

    if not args.no_bwd:
        out["backward"] = bench_backward(w, stream, x, dt, A, B, C, D, h0)

    if not args.no_cpu_baseline:
        from oracle import oracle
        omp = os.environ.get("OMP_NUM_THREADS")
        threads = int(omp or 0) or (os.cpu_count() or 1)

        def oracle_run(idx, nthreads):
            wi = wl.WORKLOADS[idx]
            ii = inp if idx == FWD_INDEX else wl.workload_inputs(idx)
            io = ii["io"]
            t = time.perf_counter()
            if wi["name"] == "decode":
                oracle.ssd_decode(ii["state"], wl.as_f64(ii["x"], io), ii["dt"], ii["A"], wl.as_f64(ii["B"], io),
                                  wl.as_f64(ii["C"], io), ii["D"], nthreads=nthreads)
                ntok = wi["batch"]
            else:
                oracle.ssd_fwd(wl.as_f64(ii["x"], io), ii["dt"], ii["A"], wl.as_f64(ii["B"], io),
                               wl.as_f64(ii["C"], io), ii["D"], init_state=ii.get("init_state"),
                               cu_seqlens=ii.get("cu_seqlens"), nthreads=nthreads)
                ntok = ii["x"].shape[0] * ii["x"].shape[1]
            return ntok, time.perf_counter() - t

        ntok, cpu_s = oracle_run(FWD_INDEX, threads)
        one_core = {}
        for idx in (0, 1, 4):      # median of three single-thread runs
            runs = [oracle_run(idx, 1) for _ in range(3)]
            med = sorted(r[1] for r in runs)[1]
            one_core[wl.WORKLOADS[idx]["name"]] = {"tokens_per_s": runs[0][0] / med, "s": med}
        n3, s3 = oracle_run(3, threads)
        out["cpu_baseline"] = {"value": ntok / cpu_s, "unit": "tokens/s", "cores": threads,
                               "kind": "oracle",
                               "sample": "the whole 2.7B-layer workload (4 x 8192 tokens, 80 heads), fp64 "
                                         f"sequential recurrence, one run, {cpu_s:.2f} s",
                               "cpu_model": cpu_model(), "omp_num_threads": omp, "logical_cpus": os.cpu_count(),
                               "varlen_packed_all_cores": {"tokens_per_s": n3 / s3, "s": s3},
                               "one_core": one_core}
    print(json.dumps(out))


if __name__ == "__main__":
    main()

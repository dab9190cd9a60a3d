"""Benchmark of the fused causal FFT convolution on one MI355X.

One step = one lconv_fftconv_fwd call over the whole synthetic batch (load, gate, forward
transform, spectral product, inverse transform, truncation, skip, gate, store).  The filter
spectrum is computed once beforehand (timed separately).  Prints ONE JSON line.

The gradient call (lconv_fftconv_bwd: du, dq, dv, dk, dD from a seeded dy) is timed the same
way on the same inputs and reported in the line's "backward" object (sequence lengths it
supports, N <= 4096); it is not part of the step.

Timing: W warm-up steps, then exactly K steps between two synchronizations, bracketed by one
event pair on the launch stream and preceded by a bounded spin kernel so the GPU runs the K
kernels back to back (ms_per_step = event time / K; the host wall time is reported beside it).
The "timing" object adds per-launch median / min / p90, back to back and after a 512 MiB cache
scrub.

Algorithmic bytes (what the method must move): (n_in + 1) * B*H*N * s for the activations
(n_in = 3 gated, 1 otherwise), plus the filter spectrum once at its minimal size
H*(N+1)*2*s (Hermitian half in the I/O dtype), plus D.  Nominal flops per row:
2 * 2.5 M log2 M + 6 (N+1) + g N with M = 2N (g = 4 gated, 2 otherwise).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}   # dense TFLOP/s
METRIC = "fftconv GB/s, TFLOP/s, %roofline at B16\u00b7H768\u00b7N4096 bf16 causal, 1 GPU"
# Hardware-counter summaries (rocprofv3 FETCH_SIZE / WRITE_SIZE scaled by a plain copy, and the
# matrix-core op count) per workload; they carry the hash of the kernel sources they were taken
# on and are ignored once those sources change.
COUNTER_FILES = {"hyena_gated_bf16_b16_h768_n4096": "profiles/conv8k_hyena_gated_bf16_b16_h768_n4096_counters.md"}
KERNEL_SOURCES = ("fft_long_convolution_amd/csrc/fused1d_kernels.h", "fft_long_convolution_amd/csrc/fused1d_conv.hip",
                  "fft_long_convolution_amd/csrc/fused_io.h", "fft_long_convolution_amd/csrc/lconv_device.h")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_summary(workload):
    """Key/value lines of the workload's counter summary, or {} when absent or stale."""
    path = COUNTER_FILES.get(workload)
    if not path or not os.path.exists(os.path.join(ROOT, path)):
        return {}
    import re
    kv = {}
    for line in open(os.path.join(ROOT, path)):
        m = re.match(r"^([a-z0-9_]+): (\S+)\s*$", line)
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("source_sha256") != kernel_source_hash():
        return {}
    kv["path"] = path
    return kv


def algorithmic_bytes(spec):
    s = {"f32": 4, "f16": 2, "bf16": 2}[spec.dtype]
    if spec.kind == "2d":
        P = 2 * spec.S
        act = 2 * spec.B * spec.C * spec.S * spec.S * s
        kf = spec.C * P * (P // 2 + 1) * 2 * s
        return act + kf + spec.C * s
    if spec.kind == "3d":
        P = 2 * spec.S
        act = 2 * spec.B * spec.C * spec.S ** 3 * s
        kf = spec.C * P * P * (P // 2 + 1) * 2 * s
        return act + kf + spec.C * s
    n_in = 3 if spec.gated else 1
    act = (n_in + 1) * spec.B * spec.H * spec.N * s
    kf = spec.H * (spec.taps + 1) * 2 * s          # the filter's spectrum: taps, not N
    if spec.name.startswith("ssm_"):               # the filter is its modes: nothing of length N
        kf = 0
    return act + kf + spec.H * s


def backward_bytes(spec):
    """Least data the gradient call must move: read dy, u and the gates, write du and one
    output per gate, read the filter spectrum (Hermitian half) and D, write dk and dD (fp32)."""
    s = {"f32": 4, "f16": 2, "bf16": 2}[spec.dtype]
    act = spec.B * spec.H * spec.N * s
    g = 2 if spec.gated else 0
    return (2 + g) * act + (1 + g) * act + spec.H * (spec.N + 1) * 2 * s + spec.H * s + \
        spec.H * (spec.N + 1) * 4


def nominal_flops(spec):
    if spec.kind == "2d":
        P = 2 * spec.S
        per = 2 * 2.5 * P * P * math.log2(P * P) + 6 * P * (P // 2 + 1) + 2 * spec.S ** 2
        return per * spec.B * spec.C
    if spec.kind == "3d":
        P = 2 * spec.S
        per = 2 * 2.5 * P ** 3 * math.log2(P ** 3) + 6 * P * P * (P // 2 + 1) + 2 * spec.S ** 3
        return per * spec.B * spec.C
    g = 4 if spec.gated else 2
    if spec.L:  # partial: one transform pair of length M = 2 C per block of C outputs
        M = 512
        while M < 2 * spec.L:
            M *= 2
        blocks = -(-spec.N // (M // 2))
        per = blocks * (2 * 2.5 * M * math.log2(M) + 6 * (M // 2 + 1)) + g * spec.N
        return per * spec.B * spec.H
    M = 2 * spec.N
    per = 2 * 2.5 * M * math.log2(M) + 6 * (spec.N + 1) + g * spec.N
    return per * spec.B * spec.H


def to_dev(a, dtype):
    import torch
    if a is None:
        return None
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def cpu_baseline(d, budget_s=12.0):
    """The float64 oracle on a bounded sample of the same workload (full rows)."""
    import oracle
    spec = d["spec"]
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(cores, 16))
    dt = {"f32": oracle.DT_F32, "f16": oracle.DT_F16, "bf16": oracle.DT_BF16}[spec.dtype]
    s = {"f32": 4, "f16": 2, "bf16": 2}[spec.dtype]
    rng = np.random.default_rng(9)
    if spec.kind == "2d":
        raise NotImplementedError
    n_in = 3 if spec.gated else 1
    if spec.L:  # short filter: single positions (each costs L multiply-adds)
        npts = 4096
        while True:
            pts = np.stack([rng.integers(0, spec.B, npts), rng.integers(0, spec.H, npts),
                            rng.integers(0, spec.N, npts)], 1)
            t0 = time.perf_counter()
            oracle.conv1d_short_points(d["u"], d["k"], d["D"], pts, q=d["q"], v=d["v"], dt=dt,
                                       nthreads=cores)
            el = time.perf_counter() - t0
            if el >= budget_s or npts >= 1 << 26:
                break
            npts = int(max(npts * 2, npts * budget_s / max(el, 1e-3) * 1.05))
        gbs = npts * (n_in + 1) * s / el / 1e9
        return {"value": round(gbs, 6), "unit": "GB/s", "cores": cores, "kind": "oracle",
                "sample": f"{npts} output positions of {spec.name}, direct float64 window sums, "
                          f"{el:.1f} s"}
    row_bytes = (n_in + 1) * spec.N * s
    # calibrate on a few rows, then size the sample for about budget_s seconds
    nrows = cores
    while True:
        rows = np.stack([rng.integers(0, spec.B, nrows), rng.integers(0, spec.H, nrows)], 1)
        t0 = time.perf_counter()
        oracle.conv1d_rows(d["u"], d["k"], d["D"], rows, q=d["q"], v=d["v"], dt=dt, nthreads=cores)
        el = time.perf_counter() - t0
        if el >= budget_s or nrows >= spec.B * spec.H:
            break
        nrows = int(min(spec.B * spec.H, max(nrows * 2, nrows * budget_s / max(el, 1e-3) * 1.05)))
    gbs = nrows * row_bytes / el / 1e9
    return {"value": round(gbs, 6), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{nrows} full rows (b,h) of {spec.name}, direct float64 sum, {el:.1f} s"}


def prime(launches):
    """Queue a bounded spin kernel (about 25 us of GPU time per launch to follow) on the current
    stream, so that the GPU is still busy when the host has queued the next launches."""
    import torch
    torch.cuda._sleep(int(50_000 * max(launches, 1)))


def _stats_us(ms):
    a = np.sort(np.asarray(ms, np.float64)) * 1e3
    return {"median": round(float(np.median(a)), 3), "min": round(float(a[0]), 3),
            "p90": round(float(np.percentile(a, 90)), 3)}


def launch_distribution(step, args):
    """Per-launch times after the timed region: R launches each between its own event pair,
    back to back ("hot"), then R launches each preceded by a read of a 512 MiB buffer outside
    the events ("scrubbed": the 256 MB last-level cache then holds none of the inputs; a read,
    not a write, so no dirty lines are still draining to HBM when the launch starts).  Returns
    median / min / p90 in microseconds for both, or {} with --dist 0."""
    import torch
    R = args.dist
    if R <= 0:
        return {}
    scrub = torch.ones((512 << 20) // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty((1,), dtype=torch.float32, device="cuda")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(R)]
    out = {"launches": R, "scrub_bytes": scrub.numel() * 4, "scrub": "read"}
    for mode in ("hot", "scrubbed"):
        torch.cuda.synchronize()
        prime(R)
        for i, (e0, e1) in enumerate(evs):
            if mode == "scrubbed":
                torch.sum(scrub, dim=0, keepdim=True, out=sink)
            e0.record()
            step()
            e1.record()
        torch.cuda.synchronize()
        out[mode + "_us"] = _stats_us([e0.elapsed_time(e1) for e0, e1 in evs])
    del scrub
    return out


def time_calls(call, args):
    """ms per call over K calls (after W warm-up calls), one event pair on the current stream."""
    import torch
    for _ in range(args.warmup):
        call()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    prime(3 * args.steps)
    ev0.record()
    for _ in range(args.steps):
        call()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / args.steps


def grad_report(ms, nbytes, outputs, launches, wsb):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms_per_call": round(ms, 5), "algorithmic_bytes": nbytes, "achieved": round(gbs, 2), "unit": "GB/s",
            "peak": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4), "outputs": outputs, "launches": launches,
            "workspace_bytes": wsb}


def time_backward_2d(lconv, wl, spec, u, kf, D, args):
    """The 2D gradient call (du, dk, dD) on the forward's inputs and a seeded dy.  Algorithmic
    bytes: read dy and u, write du, read the Hermitian half of the spectrum and D, write dk and dD
    (fp32)."""
    import torch
    s = 2
    dy = to_dev(wl.make_grad_2d(spec), spec.dtype)
    du = torch.empty_like(u)
    dk = torch.empty((spec.C, spec.Hs, spec.cols), dtype=torch.float32, device="cuda")
    dD = torch.empty((spec.C,), dtype=torch.float32, device="cuda")
    dtc = lconv.dtype_code(u.dtype)
    wsb = lconv.lconv_fftconv2d_bwd_workspace_bytes(spec.B, spec.C, spec.Hs, spec.cols, dtc)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        st = lconv.lconv_fftconv2d_bwd(dy.data_ptr(), u.data_ptr(), kf.data_ptr(), D.data_ptr(), du.data_ptr(),
                                       dk.data_ptr(), dD.data_ptr(), spec.B, spec.C, spec.Hs, spec.cols, dtc,
                                       ws.data_ptr(), wsb, stream.cuda_stream)
        if st != 0:
            raise lconv.LconvError(st, "lconv_fftconv2d_bwd")
    act = spec.B * spec.C * spec.Hs * spec.cols * s
    P = 2 * spec.S
    nbytes = 3 * act + spec.C * P * (P // 2 + 1) * 2 * s + spec.C * s + spec.C * spec.Hs * spec.cols * 4 + spec.C * 4
    return grad_report(time_calls(call, args), nbytes, "du (dtype); dk, dD (fp32)",
                       "adjoint spectrum; 2D kernel on dy (du); 2D kernel in spectrum mode (rotated-dy spectra); 2D kernel over B*C "
                       "one-image channels; batch sum (dk); dot (dD)", wsb)


def time_backward_partial(lconv, wl, spec, u, kf, D, q, v, args):
    """The partial convolution's gradient call on the forward's inputs and a seeded dy.
    Algorithmic bytes as for the full gradient, with the spectrum and dk at the L taps."""
    import torch
    s = {"f32": 4, "f16": 2, "bf16": 2}[spec.dtype]
    L = spec.L
    dy = to_dev(wl.make_grad_1d(spec), spec.dtype)
    du = torch.empty_like(u)
    dq = torch.empty_like(u) if q is not None else None
    dv = torch.empty_like(u) if v is not None else None
    dk = torch.empty((spec.H, L), dtype=torch.float32, device="cuda")
    dD = torch.empty((spec.H,), dtype=torch.float32, device="cuda")
    dtc = lconv.dtype_code(u.dtype)
    wsb = lconv.lconv_fftconv_partial_bwd_workspace_bytes(spec.B, spec.H, spec.N, dtc)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    p = lambda t: None if t is None else t.data_ptr()

    def call():
        st = lconv.lconv_fftconv_partial_bwd(dy.data_ptr(), u.data_ptr(), kf.data_ptr(), D.data_ptr(), p(q), p(v),
                                             du.data_ptr(), p(dq), p(dv), dk.data_ptr(), dD.data_ptr(), spec.B,
                                             spec.H, spec.N, L, dtc, ws.data_ptr(), wsb, stream.cuda_stream)
        if st != 0:
            raise lconv.LconvError(st, "lconv_fftconv_partial_bwd")
    act = spec.B * spec.H * spec.N * s
    g = 2 if spec.gated else 0
    nbytes = (2 + g) * act + (1 + g) * act + spec.H * (L + 1) * 2 * s + spec.H * s + spec.H * (L + 1) * 4
    return grad_report(time_calls(call, args), nbytes, "du, dq, dv (dtype); dk [H, L], dD (fp32)",
                       "partial forward gated by dy (dv); rev(dy v); partial forward of it (dx); du, dq; "
                       "full-length filter gradient (first L lags)", wsb)


def time_backward(lconv, wl, spec, u, kf, D, q, v, args):
    """K timed gradient calls (after W warm-up calls) on the forward's inputs and a seeded dy."""
    import torch
    dy = to_dev(wl.make_grad_1d(spec), spec.dtype)
    du = torch.empty_like(u)
    dq = torch.empty_like(u) if q is not None else None
    dv = torch.empty_like(u) if v is not None else None
    dk = torch.empty((spec.H, spec.N), dtype=torch.float32, device="cuda")
    dD = torch.empty((spec.H,), dtype=torch.float32, device="cuda")
    dtc = lconv.dtype_code(u.dtype)
    stream = torch.cuda.current_stream()
    p = lambda t: None if t is None else t.data_ptr()
    wsb = lconv.lconv_fftconv_bwd_workspace_bytes(spec.B, spec.H, spec.N, dtc)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    fwsb = lconv.lconv_fftconv_workspace_bytes(spec.B, spec.H, spec.N, dtc)
    fws = torch.empty(max(fwsb, 1), dtype=torch.uint8, device="cuda")

    def call():
        st = lconv.lconv_fftconv_bwd(dy.data_ptr(), u.data_ptr(), kf.data_ptr(), D.data_ptr(), p(q),
                                     p(v), du.data_ptr(), p(dq), p(dv), dk.data_ptr(), dD.data_ptr(),
                                     spec.B, spec.H, spec.N, dtc, ws.data_ptr(), wsb, stream.cuda_stream)
        if st != 0:
            raise lconv.LconvError(st, "lconv_fftconv_bwd")
    for _ in range(args.warmup):
        call()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    prime(3 * args.steps)
    ev0.record()
    for _ in range(args.steps):
        call()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    nbytes = backward_bytes(spec)
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {"ms_per_call": round(ms, 5), "algorithmic_bytes": nbytes, "achieved": round(gbs, 2),
           "unit": "GB/s", "peak": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4),
           "outputs": "du, dq, dv (dtype); dk, dD (fp32)",
           "launches": ("forward kernel gated by dy (dv); adjoint kernel (du, dq); "
                        "filter-gradient kernel (dk, dD)") if spec.N <= 4096 else
                       ("multi-pass forward gated by dy (dv); rev(dy v); multi-pass forward of it "
                        "(dx); du, dq; filter spectra of the rows q u; multi-pass forward of rev(dy v) "
                        "with them; batch sum (dk, dD)"),
           "workspace_bytes": wsb}
    if v is not None:
        # the training pair: the forward that also saves the pre-gate output c, and the gradient
        # that takes dv = dy * c from it (one elementwise pass instead of the dy-gated transform)
        y = torch.empty_like(u)
        c = torch.empty_like(u)

        def fwd_save():
            st = lconv.lconv_fftconv_fwd_save(u.data_ptr(), kf.data_ptr(), D.data_ptr(), y.data_ptr(),
                                              c.data_ptr(), p(q), p(v), spec.B, spec.H, spec.N, dtc,
                                              fws.data_ptr(), fwsb, stream.cuda_stream)
            if st != 0:
                raise lconv.LconvError(st, "lconv_fftconv_fwd_save")

        def bwd_saved():
            st = lconv.lconv_fftconv_bwd_saved(dy.data_ptr(), u.data_ptr(), kf.data_ptr(), D.data_ptr(), p(q),
                                               p(v), c.data_ptr(), du.data_ptr(), p(dq), p(dv), dk.data_ptr(),
                                               dD.data_ptr(), spec.B, spec.H, spec.N, dtc, ws.data_ptr(), wsb,
                                               stream.cuda_stream)
            if st != 0:
                raise lconv.LconvError(st, "lconv_fftconv_bwd_saved")

        def timed(fn):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            prime(3 * args.steps)
            ev0.record()
            for _ in range(args.steps):
                fn()
            ev1.record()
            torch.cuda.synchronize()
            return ev0.elapsed_time(ev1) / args.steps

        ms_f, ms_b = timed(fwd_save), timed(bwd_saved)
        out["saved"] = {"fwd_save_ms": round(ms_f, 5), "bwd_saved_ms": round(ms_b, 5),
                        "launches": "forward kernel that also stores c; dv = dy * c (elementwise); "
                                    "adjoint kernel; filter-gradient kernel"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-bwd", action="store_true", help="skip the gradient call's timing")
    ap.add_argument("--keep", default=None,
                    help="frequency-sparse call: bit mask (e.g. 0xe000000f) of the frequency "
                         "blocks kept (f mod R); the step is lconv_fftconv_sparse_fwd")
    ap.add_argument("--butterfly", action="store_true",
                    help="learned-Butterfly call (lconv_butterfly_fwd, seeded factor blocks; "
                         "N <= 4096) instead of the FFT convolution")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--dist", type=int, default=20,
                    help="launches for the per-launch median / min / p90, hot and after a cache "
                         "scrub (0: skip)")
    ap.add_argument("--copy-calibrate", action="store_true",
                    help="run only a plain 256 MiB device copy (reads and writes 256 MiB per "
                         "launch): the reference for scaling FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.copy_calibrate:
        import torch
        x = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": 256 << 20, "launches": 5}))
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the per-(b,h) rows would shard over GPUs with no exchange, but no multi-GPU run "
              "is part of it.", file=sys.stderr)
        sys.exit(2)

    import torch
    from fft_long_convolution_amd import lconv
    from fft_long_convolution_amd import workloads as wl

    name = args.workload or wl.HEADLINE
    d = wl.make(name)
    spec = d["spec"]
    torch.cuda.set_device(0)
    dt = spec.dtype
    lconv.load()

    if spec.kind == "2d":
        u, k, D = (to_dev(d[x], dt) for x in ("u", "k", "D"))
        run_filter = lambda: lconv.filter_fft2d(k)
        kf = run_filter()
        y = torch.empty_like(u)
        step = lambda: lconv.fftconv2d(u, kf, D, out=y)
    elif spec.kind == "3d":
        u, k, D = (to_dev(d[x], dt) for x in ("u", "k", "D"))
        run_filter = lambda: lconv.filter_fft3d(k)
        kf = run_filter()
        y = torch.empty_like(u)
        dtc = lconv.dtype_code(u.dtype)
        wsb3 = lconv.lconv_fftconv3d_workspace_bytes(spec.B, spec.C, spec.S, dtc)
        ws3 = torch.empty(max(wsb3, 1), dtype=torch.uint8, device="cuda")
        stream = torch.cuda.current_stream()

        def step():
            st = lconv.lconv_fftconv3d_fwd(u.data_ptr(), kf.data_ptr(), D.data_ptr(), y.data_ptr(), spec.B,
                                           spec.C, spec.S, dtc, ws3.data_ptr(), wsb3, stream.cuda_stream)
            if st != 0:
                raise lconv.LconvError(st, "lconv_fftconv3d_fwd")
    elif spec.name.startswith("ssm_"):  # state-space filter, chunks with state passing
        NS, T = 64, 4096
        u, q, v, D = (to_dev(d[x], dt) for x in ("u", "q", "v", "D"))
        lam_h, W_h = wl.ssm_modes(spec.H, NS, seed=spec.seed + 1)
        lam_d = torch.from_numpy(lam_h.astype(np.complex64)).cuda()
        W_d = torch.from_numpy(W_h.astype(np.complex64)).cuda()
        run_filter = lambda: lconv.ssm_prepare(lam_d, W_d, T, u.dtype)
        kf = run_filter()
        y = torch.empty_like(u)
        dtc = lconv.dtype_code(u.dtype)
        wss = lconv.lconv_fftconv_ssm_workspace_bytes(spec.B, spec.H, spec.N, NS, T)
        wsd = torch.empty(max(wss, 1), dtype=torch.uint8, device="cuda")
        stream = torch.cuda.current_stream()
        p = lambda t: None if t is None else t.data_ptr()

        def step():
            st = lconv.lconv_fftconv_ssm_fwd(u.data_ptr(), kf.data_ptr(), D.data_ptr(), y.data_ptr(), p(q), p(v),
                                             spec.B, spec.H, spec.N, NS, T, dtc, wsd.data_ptr(), wss,
                                             stream.cuda_stream)
            if st != 0:
                raise lconv.LconvError(st, "lconv_fftconv_ssm_fwd")
    elif args.butterfly:  # learned Butterfly: caller factor blocks, one real row per transform
        u, q, v, k, D = (to_dev(d[x], dt) for x in ("u", "q", "v", "k", "D"))
        blocks = torch.from_numpy(wl.butterfly_blocks(spec.N, seed=spec.seed + 3)).cuda()
        tables = lconv.butterfly_tables(blocks, spec.N, u.dtype)
        run_filter = lambda: lconv.butterfly_filter(k, tables)
        kf = run_filter()
        y = torch.empty_like(u)
        dtc = lconv.dtype_code(u.dtype)
        stream = torch.cuda.current_stream()
        p = lambda t: None if t is None else t.data_ptr()

        def step():
            st = lconv.lconv_butterfly_fwd(u.data_ptr(), kf.data_ptr(), D.data_ptr(), y.data_ptr(), p(q), p(v),
                                           tables.data_ptr(), spec.B, spec.H, spec.N, dtc, stream.cuda_stream)
            if st != 0:
                raise lconv.LconvError(st, "lconv_butterfly_fwd")
    elif args.keep is not None:  # frequency-sparse convolution
        keep = int(args.keep, 0)
        u, q, v, k, D = (to_dev(d[x], dt) for x in ("u", "q", "v", "k", "D"))
        run_filter = lambda: lconv.filter_fft(k)
        kf = run_filter()
        y = torch.empty_like(u)
        dtc = lconv.dtype_code(u.dtype)
        stream = torch.cuda.current_stream()
        p = lambda t: None if t is None else t.data_ptr()

        def step():
            st = lconv.lconv_fftconv_sparse_fwd(u.data_ptr(), kf.data_ptr(), D.data_ptr(), y.data_ptr(),
                                                p(q), p(v), spec.B, spec.H, spec.N, keep, dtc,
                                                stream.cuda_stream)
            if st != 0:
                raise lconv.LconvError(st, "lconv_fftconv_sparse_fwd")
    elif spec.L:  # partial convolution: short filter, any sequence length
        u, q, v, k, D = (to_dev(d[x], dt) for x in ("u", "q", "v", "k", "D"))
        run_filter = lambda: lconv.filter_fft(k)
        kf = run_filter()
        y = torch.empty_like(u)
        dtc = lconv.dtype_code(u.dtype)
        stream = torch.cuda.current_stream()
        p = lambda t: None if t is None else t.data_ptr()

        def step():
            st = lconv.lconv_fftconv_partial_fwd(u.data_ptr(), kf.data_ptr(), D.data_ptr(), y.data_ptr(),
                                                 p(q), p(v), spec.B, spec.H, spec.N, spec.L, dtc,
                                                 stream.cuda_stream)
            if st != 0:
                raise lconv.LconvError(st, "lconv_fftconv_partial_fwd")
    else:
        u, q, v, k, D = (to_dev(d[x], dt) for x in ("u", "q", "v", "k", "D"))
        run_filter = lambda: lconv.filter_fft(k)
        kf = run_filter()
        y = torch.empty_like(u)
        wsb = lconv.lconv_fftconv_workspace_bytes(spec.B, spec.H, spec.N, lconv.dtype_code(u.dtype))
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
        dtc = lconv.dtype_code(u.dtype)
        stream = torch.cuda.current_stream()

        def step():
            st = lconv.lconv_fftconv_fwd(u.data_ptr(), kf.data_ptr(), D.data_ptr(), y.data_ptr(),
                                         None if q is None else q.data_ptr(),
                                         None if v is None else v.data_ptr(),
                                         spec.B, spec.H, spec.N, dtc,
                                         ws.data_ptr() if wsb else None, wsb, stream.cuda_stream)
            if st != 0:
                raise lconv.LconvError(st, "lconv_fftconv_fwd")

    torch.cuda.synchronize()
    # filter spectrum timing (not part of a step)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    kf2 = run_filter()
    e1.record()
    torch.cuda.synchronize()
    filter_ms = e0.elapsed_time(e1)
    del kf2

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Timed region: exactly K steps between two synchronizations.  One event pair on the launch
    # stream (torch's current stream, which the library is given) brackets the K launches.  A
    # bounded spin kernel queued first keeps the GPU busy while the host queues the region, so
    # the first launch does not wait on the host and the events time the K kernels back to
    # back: the step time is the event time / K, the same quantity a kernel trace averages.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    prime(args.steps)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = avg_ms

    timing = launch_distribution(step, args)

    nbytes = algorithmic_bytes(spec)
    flops = nominal_flops(spec)
    if args.keep is not None:  # only the kept blocks of the filter spectrum are needed
        R = lconv.lconv_freq_blocks(spec.N)
        frac = bin(int(args.keep, 0) & ((1 << R) - 1)).count("1") / R
        s_ = {"f32": 4, "f16": 2, "bf16": 2}[dt]
        nbytes -= int(round((1 - frac) * spec.H * (spec.N + 1) * 2 * s_))
    elems = spec.B * (spec.H if spec.kind == "1d" else spec.C) * \
        {"1d": getattr(spec, "N", 0), "2d": getattr(spec, "S", 0) ** 2, "3d": getattr(spec, "S", 0) ** 3}[spec.kind]
    gbs = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (avg_ms * 1e-3) / 1e9

    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "host_wall_ms": round(wall * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": {"workload": spec.name, "B": spec.B, **({"L": spec.L} if getattr(spec, "L", 0) else {}),
                   **({"keep": args.keep} if args.keep is not None else {}),
                   **({"learned_butterfly": True} if args.butterfly else {}),
                   ("H" if spec.kind == "1d" else "C"): (spec.H if spec.kind == "1d" else spec.C),
                   ("N" if spec.kind == "1d" else "S"): (spec.N if spec.kind == "1d" else spec.S),
                   "gated": bool(getattr(spec, "gated", False)), "parallelism": "none"},
        "tflops": round(flops / (ms_per_step * 1e-3) / 1e12, 3),
        "elements_per_s": float("%.4g" % (elems / (ms_per_step * 1e-3))),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "filter_fft_ms": round(filter_ms, 4),
        "algorithmic_bytes": nbytes,
        "nominal_flops": flops,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "kernel_avg_us": round(avg_ms * 1e3, 3)},
    }
    if timing:
        out["timing"] = timing
        out["timing"]["region_avg_us"] = round(avg_ms * 1e3, 3)
    cs = counter_summary(spec.name) if args.keep is None and not args.butterfly else {}  # of the FFT call
    if cs:
        out["roofline"]["traffic"] = int(float(cs["traffic_bytes_per_launch"]))
        # matrix-core GFLOP executed per launch (op counter x 512), over this run's kernel time
        mf = float(cs["mfma_gflop_executed_per_launch"]) * 1e9 / (avg_ms * 1e-3) / 1e12
        out["mfma"] = {"executed_tflops": round(mf, 1), "peak": MFMA_PEAK[dt],
                       "util": round(mf / MFMA_PEAK[dt], 4), "counters": cs["path"]}
    if not args.no_bwd and spec.kind == "1d" and spec.N % 8 == 0 and not spec.L and args.keep is None \
            and not args.butterfly and not spec.name.startswith("ssm_"):
        out["backward"] = time_backward(lconv, wl, spec, u, kf, D, q, v, args)
    elif not args.no_bwd and spec.kind == "2d":
        out["backward"] = time_backward_2d(lconv, wl, spec, u, kf, D, args)
    elif not args.no_bwd and spec.kind == "1d" and spec.L and args.keep is None and not args.butterfly:
        out["backward"] = time_backward_partial(lconv, wl, spec, u, kf, D, q, v, args)
    if not args.no_cpu and spec.kind == "1d" and not spec.name.startswith("ssm_") and not args.butterfly:
        out["cpu_baseline"] = cpu_baseline(d, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""GPU parity of the gradients: lconv_fftconv_bwd through the C ABI against the float64 oracle
(oracle.conv1d_bwd_rows for du, dq, dv; oracle.conv1d_bwd_dk for dk, dD).

Tolerance, as for the forward: max relative L2 error 1e-4 for fp32 inputs and 2e-2 for bf16 /
fp16 inputs, per (b, h) row of du, dq, dv and per channel row of dk; dD as one vector over
channels.  dD must equal dk[:, 0] exactly (the kernel stores the same value twice).  Any
non-finite output fails.
"""
import numpy as np
import pytest

import oracle
from fft_long_convolution_amd import workloads as wl
from tests.gpu_util import DT_ORACLE, TOL, from_dev, rel_l2, rel_l2_rows, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lc():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fft_long_convolution_amd import lconv
    lconv.load()
    return lconv


def inputs(spec, gates):
    d = wl.make(spec)
    dy = wl.make_grad_1d(spec)
    q = d["q"] if "q" in gates else None
    v = d["v"] if "v" in gates else None
    return d, dy, q, v


def run_bwd(lc, d, dy, q, v, need_dk=True):
    import torch
    dt = d["dtype"]
    kf = lc.filter_fft(to_dev(d["k"], dt))
    out = lc.fftconv_bwd(to_dev(dy, dt), to_dev(d["u"], dt), kf, to_dev(d["D"], dt),
                         q=to_dev(q, dt), v=to_dev(v, dt), need_dk=need_dk)
    torch.cuda.synchronize()
    du, dq, dv, dk, dD = out
    conv = lambda t: None if t is None else from_dev(t, dt)
    f32 = lambda t: None if t is None else t.cpu().numpy().astype(np.float64)
    return conv(du), conv(dq), conv(dv), f32(dk), f32(dD)


def check_rows(got, d, dy, q, v, rows, nthreads):
    """du, dq, dv on the given (b, h) rows against the oracle; returns the max errors."""
    dt = d["dtype"]
    du, dq, dv = got
    r_du, r_dq, r_dv = oracle.conv1d_bwd_rows(d["u"], d["k"], d["D"], dy, rows, q=q, v=v,
                                              dt=DT_ORACLE[dt], nthreads=nthreads)
    bi = np.asarray([r[0] for r in rows])
    hi = np.asarray([r[1] for r in rows])
    errs = {}
    for name, g, r in (("du", du, r_du), ("dq", dq, r_dq), ("dv", dv, r_dv)):
        if r is None:
            assert g is None, name
            continue
        gg = g[bi, hi]
        assert np.all(np.isfinite(gg)), name
        errs[name] = float(rel_l2_rows(gg, r).max())
    return errs


def check_dk(dk, dD, d, dy, q, v, chans, nthreads):
    dt = d["dtype"]
    r_dk, r_dD = oracle.conv1d_bwd_dk(d["u"], dy, chans, q=q, v=v, dt=DT_ORACLE[dt], nthreads=nthreads)
    g = dk[np.asarray(chans)]
    assert np.all(np.isfinite(g)) and np.all(np.isfinite(dD))
    assert np.array_equal(dD, dk[:, 0]), "dD must be the stored dk[:, 0]"
    return {"dk": float(rel_l2_rows(g, r_dk).max()), "dD": rel_l2(dD[np.asarray(chans)], r_dD)}


SWEEP_N = [8, 64, 120, 256, 1000, 1024, 2048, 4096]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("N", SWEEP_N)
@pytest.mark.parametrize("B,gates", [(1, ""), (3, "qv"), (4, "q"), (2, "v")])
def test_bwd_sweep_full(lc, nthreads, dtype, N, B, gates):
    H = 3
    spec = wl.spec_1d(B, H, N, dtype, gated=True, seed=300 + N + B)
    say(f"[bwd sweep] dtype={dtype} B={B} H={H} N={N} gates={gates!r} seed={spec.seed}")
    d, dy, q, v = inputs(spec, gates)
    du, dq, dv, dk, dD = run_bwd(lc, d, dy, q, v)
    rows = [(b, h) for b in range(B) for h in range(H)]
    errs = check_rows((du, dq, dv), d, dy, q, v, rows, nthreads)
    errs.update(check_dk(dk, dD, d, dy, q, v, list(range(H)), nthreads))
    say("   " + " ".join(f"{k}={e:.3e}" for k, e in errs.items()) + f" (tol {TOL[dtype]})")
    for k, e in errs.items():
        assert e <= TOL[dtype], (k, e)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_many_channels_ragged(lc, nthreads, dtype):
    """More channels than workgroups hold at once, an odd batch and a length that does not fill
    the half transform: several channels per workgroup and a ragged last group."""
    B, H, N = 5, 300, 1000
    spec = wl.spec_1d(B, H, N, dtype, gated=True, seed=4242)
    say(f"[bwd ragged] dtype={dtype} B={B} H={H} N={N} seed={spec.seed}")
    d, dy, q, v = inputs(spec, "qv")
    du, dq, dv, dk, dD = run_bwd(lc, d, dy, q, v)
    rng = np.random.default_rng(7)
    rows = [(int(b), int(h)) for b, h in zip(rng.integers(0, B, 24), rng.integers(0, H, 24))]
    rows += [(B - 1, H - 1), (0, 0)]
    errs = check_rows((du, dq, dv), d, dy, q, v, rows, nthreads)
    chans = sorted(set([0, 1, H - 1] + [int(h) for h in rng.integers(0, H, 13)]))
    errs.update(check_dk(dk, dD, d, dy, q, v, chans, nthreads))
    say("   " + " ".join(f"{k}={e:.3e}" for k, e in errs.items()))
    for k, e in errs.items():
        assert e <= TOL[dtype], (k, e)


def test_bwd_hyena_workload_sampled(lc, nthreads):
    """The gated bf16 workload at full size (B16 H768 N4096): sampled rows and channels."""
    spec = wl.WORKLOADS["hyena_gated_bf16_b16_h768_n4096"]
    say(f"[bwd hyena] {spec.name} seed={spec.seed}")
    d, dy, q, v = inputs(spec, "qv")
    du, dq, dv, dk, dD = run_bwd(lc, d, dy, q, v)
    B, H = spec.B, spec.H
    rng = np.random.default_rng(11)
    rows = [(int(b), int(h)) for b, h in zip(rng.integers(0, B, 10), rng.integers(0, H, 10))]
    rows += [(B - 1, H - 1)]
    errs = check_rows((du, dq, dv), d, dy, q, v, rows, nthreads)
    chans = sorted(set([0, H - 1] + [int(h) for h in rng.integers(0, H, 4)]))
    errs.update(check_dk(dk, dD, d, dy, q, v, chans, nthreads))
    say("   " + " ".join(f"{k}={e:.3e}" for k, e in errs.items()))
    for k, e in errs.items():
        assert e <= TOL["bf16"], (k, e)


def test_bwd_without_filter_gradient(lc, nthreads):
    spec = wl.spec_1d(3, 2, 512, "bf16", gated=True, seed=77)
    say(f"[bwd no-dk] seed={spec.seed}")
    d, dy, q, v = inputs(spec, "qv")
    du, dq, dv, dk, dD = run_bwd(lc, d, dy, q, v, need_dk=False)
    assert dk is None and dD is None
    errs = check_rows((du, dq, dv), d, dy, q, v, [(b, h) for b in range(3) for h in range(2)], nthreads)
    for k, e in errs.items():
        assert e <= TOL["bf16"], (k, e)


def test_bwd_empty_batch_zeroes_filter_gradient(lc):
    import torch
    H, N = 4, 64
    say("[bwd B=0]")
    dk = torch.full((H, N), 7.0, device="cuda")
    dD = torch.full((H,), 7.0, device="cuda")
    st = lc.lconv_fftconv_bwd(None, None, None, None, None, None, None, None, None,
                              dk.data_ptr(), dD.data_ptr(), 0, H, N, lc.BF16, None, 0,
                              torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert float(dk.abs().max()) == 0.0 and float(dD.abs().max()) == 0.0


# ---- sequences past one workgroup: the multi-pass gradient ----------------------------------

LONG_N = [8192, 16384, 40960]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("N", LONG_N)
@pytest.mark.parametrize("B,gates", [(3, "qv"), (2, ""), (1, "q")])
def test_bwd_long_full(lc, nthreads, dtype, N, B, gates):
    """N > 4096 (chunked multi-pass transforms): every row of du, dq, dv and every channel of
    dk, dD against the oracle."""
    H = 2
    spec = wl.spec_1d(B, H, N, dtype, gated=True, seed=700 + N + B, decay=1e-4)
    say(f"[bwd long] dtype={dtype} B={B} H={H} N={N} gates={gates!r} seed={spec.seed}")
    d, dy, q, v = inputs(spec, gates)
    du, dq, dv, dk, dD = run_bwd(lc, d, dy, q, v)
    rows = [(b, h) for b in range(B) for h in range(H)]
    errs = check_rows((du, dq, dv), d, dy, q, v, rows, nthreads)
    errs.update(check_dk(dk, dD, d, dy, q, v, list(range(H)), nthreads))
    say("   " + " ".join(f"{k}={e:.3e}" for k, e in errs.items()) + f" (tol {TOL[dtype]})")
    for k, e in errs.items():
        assert e <= TOL[dtype], (k, e)


def _sampled_bwd(lc, nthreads, d, dy, q, v, n_pts=768, n_dk=192, seed=0):
    """Pooled relative L2 of du, dq, dv at sampled (b,h,t) and of dk at sampled (h,tau), with the
    first and last positions of rows and of multi-pass chunk boundaries always included."""
    spec = d["spec"]
    B, H, N, dt = spec.B, spec.H, spec.N, spec.dtype
    du, dq, dv, dk, dD = run_bwd(lc, d, dy, q, v)
    rng = np.random.default_rng(seed)
    pts = np.stack([rng.integers(0, B, n_pts), rng.integers(0, H, n_pts), rng.integers(0, N, n_pts)], 1)
    special = [0, 1, N - 2, N - 1, 8191, 8192, N // 2 - 1, N // 2]
    pts[:len(special), 2] = special
    r_du, r_dq, r_dv = oracle.conv1d_bwd_points(d["u"], d["k"], d["D"], dy, pts, q=q, v=v,
                                                dt=DT_ORACLE[dt], nthreads=nthreads)
    errs = {}
    for name, g, r in (("du", du, r_du), ("dq", dq, r_dq), ("dv", dv, r_dv)):
        if r is None:
            assert g is None
            continue
        gg = g[pts[:, 0], pts[:, 1], pts[:, 2]]
        assert np.all(np.isfinite(gg)), name
        errs[name] = rel_l2(gg, r)
    kp = np.stack([rng.integers(0, H, n_dk), rng.integers(0, N, n_dk)], 1)
    kp[:len(special), 1] = special
    r_dk = oracle.conv1d_bwd_dk_points(d["u"], dy, kp, q=q, v=v, dt=DT_ORACLE[dt], nthreads=nthreads)
    gk = dk[kp[:, 0], kp[:, 1]]
    assert np.all(np.isfinite(gk)) and np.array_equal(dD, dk[:, 0])
    errs["dk"] = rel_l2(gk, r_dk)
    return errs


def test_bwd_long_workload_shape_sampled(lc, nthreads):
    """The 64K workload's shape (B4 H256 N65536, fp16, ungated), sampled, plus a gated variant
    at the same length with fewer channels."""
    spec = wl.WORKLOADS["long_f16_b4_h256_n65536"]
    say(f"[bwd 64K] {spec.name} seed={spec.seed}")
    d, dy, q, v = inputs(spec, "")
    errs = _sampled_bwd(lc, nthreads, d, dy, q, v, seed=1)
    say("   " + " ".join(f"{k}={e:.3e}" for k, e in errs.items()))
    for k, e in errs.items():
        assert e <= TOL["f16"], (k, e)
    spec2 = wl.spec_1d(3, 4, 65536, "bf16", gated=True, seed=7001, decay=1e-4)
    say(f"[bwd 64K gated] B=3 H=4 seed={spec2.seed}")
    d, dy, q, v = inputs(spec2, "qv")
    errs = _sampled_bwd(lc, nthreads, d, dy, q, v, seed=2)
    say("   " + " ".join(f"{k}={e:.3e}" for k, e in errs.items()))
    for k, e in errs.items():
        assert e <= TOL["bf16"], (k, e)


def test_bwd_very_long_sampled(lc, nthreads):
    """2^21 (the very long workload's shape, B1 H64 bf16), sampled positions."""
    spec = wl.WORKLOADS["very_long_bf16_b1_h64_n2097152"]
    say(f"[bwd 2M] {spec.name} seed={spec.seed}")
    d, dy, q, v = inputs(spec, "")
    errs = _sampled_bwd(lc, nthreads, d, dy, q, v, n_pts=256, n_dk=96, seed=3)
    say("   " + " ".join(f"{k}={e:.3e}" for k, e in errs.items()))
    for k, e in errs.items():
        assert e <= TOL["bf16"], (k, e)


@pytest.mark.parametrize("B,H,N,dtype,gates", [(2, 2, 1100000, "bf16", "qv"), (3, 1, 600000, "f16", "q")])
def test_bwd_long_row_spectra_sampled(lc, nthreads, B, H, N, dtype, gates):
    """Column lengths M1 = 512 and 256 with batch rows and gates: the filter gradient takes the
    spectra of x = q (.) u in the 16-bit compute type, gated inside the forward column pass, for the
    half rows only (B = 2 pairs rows of one channel; B = 3 ends on a lone row)."""
    spec = wl.spec_1d(B, H, N, dtype, gated=True, seed=7200 + B, decay=1e-5)
    say(f"[bwd long spectra] dtype={dtype} B={B} H={H} N={N} gates={gates!r} seed={spec.seed}")
    d, dy, q, v = inputs(spec, gates)
    errs = _sampled_bwd(lc, nthreads, d, dy, q, v, n_pts=256, n_dk=96, seed=4)
    say("   " + " ".join(f"{k}={e:.3e}" for k, e in errs.items()) + f" (tol {TOL[dtype]})")
    for k, e in errs.items():
        assert e <= TOL[dtype], (k, e)


def test_training_pair_long(lc, nthreads):
    """The training pair past one workgroup: fftconv_save's y equals the plain forward call's, c is
    the pre-gate output, and the saved-output gradient equals the plain gradient."""
    import torch
    B, H, N, dt = 3, 2, 16384, "bf16"
    spec = wl.spec_1d(B, H, N, dt, gated=True, seed=7100, decay=1e-4)
    say(f"[train pair long] B={B} H={H} N={N} seed={spec.seed}")
    d, dy, q, v = inputs(spec, "qv")
    u_, q_, v_, D_, dy_ = (to_dev(x, dt) for x in (d["u"], q, v, d["D"], dy))
    kf = lc.filter_fft(to_dev(d["k"], dt))
    y_ref = lc.fftconv(u_, kf, D_, q=q_, v=v_)
    y, c = lc.fftconv_save(u_, kf, D_, q=q_, v=v_)
    c_ref = lc.fftconv(u_, kf, D_, q=q_)
    plain = lc.fftconv_bwd(dy_, u_, kf, D_, q=q_, v=v_)
    saved = lc.fftconv_bwd(dy_, u_, kf, D_, q=q_, v=v_, c=c)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), c_ref.view(torch.int16))
    # y = v * c rounds once from the rounded c; the plain call rounds v * c from fp32
    assert rel_l2(from_dev(y, dt), from_dev(y_ref, dt)) <= 1e-2
    for name, a, b in zip(("du", "dq"), saved[:2], plain[:2]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
    assert torch.equal(saved[3], plain[3]) and torch.equal(saved[4], plain[4])
    rows = [(b, h) for b in range(B) for h in range(H)]
    errs = check_rows(tuple(from_dev(t, dt) if t is not None else None for t in saved[:3]), d, dy, q, v, rows,
                      nthreads)
    say("   " + " ".join(f"{k}={e:.3e}" for k, e in errs.items()))
    for k, e in errs.items():
        assert e <= TOL[dt], (k, e)

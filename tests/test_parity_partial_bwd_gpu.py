"""GPU parity of the partial convolution's gradients: lconv_fftconv_partial_bwd through the C ABI
against the float64 oracle (oracle.conv1d_short_bwd_rows / _dk, pinned element by element in
tests/test_oracle_short_bwd.py).

Tolerance as for the forward: max relative L2 error 1e-4 for fp32 inputs and 2e-2 for bf16 /
fp16 inputs, per (b, h) row of du, dq, dv and per channel row of dk [H, L]; dD as one vector over
channels and equal to dk[:, 0].  Any non-finite output fails.
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


def run_pbwd(lc, d, dy, q, v, need_dk=True):
    import torch
    dt = d["dtype"]
    L = d["k"].shape[1]
    kf = lc.filter_fft(to_dev(d["k"], dt))
    out = lc.fftconv_partial_bwd(to_dev(dy, dt), to_dev(d["u"], dt), kf, to_dev(d["D"], dt), L,
                                 q=to_dev(q, dt), v=to_dev(v, dt), need_dk=need_dk)
    torch.cuda.synchronize()
    du, dq, dv, dk, dD = out
    conv = lambda t: None if t is None else from_dev(t, dt)
    f32 = lambda t: None if t is None else t.cpu().numpy().astype(np.float64)
    return conv(du), conv(dq), conv(dv), f32(dk), f32(dD)


# (B, H, N, L, gates): N below, at and above L; single-pass and multi-pass lengths of N
CASES = [
    (2, 3, 1000, 64, "qv"),
    (3, 2, 256, 1000, "qv"),      # L > N: lags >= N are zero
    (2, 2, 4096, 4096, "q"),      # L = N
    (1, 2, 520, 512, "v"),        # N barely past one block
    (2, 2, 10000, 1000, "qv"),    # N on the multi-pass path
    (1, 2, 16384, 4096, ""),
    (3, 1, 8192, 200, "qv"),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("B,H,N,L,gates", CASES)
def test_partial_bwd_full(lc, nthreads, dtype, B, H, N, L, gates):
    spec = wl.spec_partial(B, H, N, L, dtype, gated=True, seed=900 + N + L + B)
    say(f"[partial bwd] dtype={dtype} B={B} H={H} N={N} L={L} gates={gates!r} seed={spec.seed}")
    d, dy, q, v = inputs(spec, gates)
    du, dq, dv, dk, dD = run_pbwd(lc, d, dy, q, v)
    rows = [(b, h) for b in range(B) for h in range(H)]
    r_du, r_dq, r_dv = oracle.conv1d_short_bwd_rows(d["u"], d["k"], d["D"], dy, rows, q=q, v=v,
                                                    dt=DT_ORACLE[dtype], nthreads=nthreads)
    errs = {}
    for name, g, r in (("du", du, r_du), ("dq", dq, r_dq), ("dv", dv, r_dv)):
        if r is None:
            assert g is None, name
            continue
        gg = g.reshape(B * H, N)
        assert np.all(np.isfinite(gg)), name
        errs[name] = float(rel_l2_rows(gg, r).max())
    r_dk, r_dD = oracle.conv1d_short_bwd_dk(d["u"], dy, list(range(H)), L, q=q, v=v, dt=DT_ORACLE[dtype],
                                            nthreads=nthreads)
    assert dk.shape == (H, L)
    assert np.all(np.isfinite(dk)) and np.all(np.isfinite(dD))
    assert np.array_equal(dD, dk[:, 0]), "dD must be the stored dk[:, 0]"
    if L > N:
        assert np.all(dk[:, N:] == 0.0)
    errs["dk"] = float(rel_l2_rows(dk, r_dk).max())
    errs["dD"] = rel_l2(dD, r_dD)
    say("   " + " ".join(f"{k}={e:.3e}" for k, e in errs.items()) + f" (tol {TOL[dtype]})")
    for k, e in errs.items():
        assert e <= TOL[dtype], (k, e)


def test_partial_bwd_long_workload_sampled(lc, nthreads):
    """The 2^21-long sequence with a 4096-tap filter (B1 H64, bf16, its gates): sampled du, dq, dv
    positions (block boundaries included) and sampled dk lags."""
    spec = wl.WORKLOADS["partial_bf16_b1_h64_n2097152_l4096"]
    say(f"[partial bwd long] {spec.name} seed={spec.seed}")
    d, dy, q, v = inputs(spec, "qv")
    du, dq, dv, dk, dD = run_pbwd(lc, d, dy, q, v)
    B, H, N, L = spec.B, spec.H, spec.N, d["k"].shape[1]
    rng = np.random.default_rng(77)
    n_pts = 256
    pts = np.stack([rng.integers(0, B, n_pts), rng.integers(0, H, n_pts), rng.integers(0, N, n_pts)], 1)
    special = [0, 1, 4095, 4096, 8191, 8192, N - 4097, N - 4096, N - 2, N - 1]
    pts[:len(special), 2] = special
    r_du, r_dq, r_dv = oracle.conv1d_short_bwd_points(d["u"], d["k"], d["D"], dy, pts, q=q, v=v,
                                                      dt=DT_ORACLE["bf16"], nthreads=nthreads)
    errs = {}
    for name, g, r in (("du", du, r_du), ("dq", dq, r_dq), ("dv", dv, r_dv)):
        if r is None:   # the workload's gates (absent ones have no gradient)
            assert g is None, name
            continue
        gg = g[pts[:, 0], pts[:, 1], pts[:, 2]]
        assert np.all(np.isfinite(gg)), name
        errs[name] = rel_l2(gg, r)
    kp = np.stack([rng.integers(0, H, 64), rng.integers(0, L, 64)], 1)
    kp[:4, 1] = [0, 1, L - 2, L - 1]
    r_dk = oracle.conv1d_short_bwd_dk_points(d["u"], dy, kp, L, q=q, v=v, dt=DT_ORACLE["bf16"], nthreads=nthreads)
    gk = dk[kp[:, 0], kp[:, 1]]
    assert np.all(np.isfinite(gk)) and np.array_equal(dD, dk[:, 0])
    errs["dk"] = rel_l2(gk, r_dk)
    say("   " + " ".join(f"{k}={e:.3e}" for k, e in errs.items()))
    for k, e in errs.items():
        assert e <= TOL["bf16"], (k, e)


def test_partial_bwd_matches_full_gradient_when_L_is_N(lc):
    """With L = N the partial gradient is the full-length gradient (dk of the same length)."""
    import torch
    spec = wl.spec_partial(3, 2, 2048, 2048, "f32", gated=True, seed=41)
    say(f"[partial bwd vs full] seed={spec.seed}")
    d, dy, q, v = inputs(spec, "qv")
    got = run_pbwd(lc, d, dy, q, v)
    kf = lc.filter_fft(to_dev(d["k"], "f32"))
    ref = lc.fftconv_bwd(to_dev(dy, "f32"), to_dev(d["u"], "f32"), kf, to_dev(d["D"], "f32"),
                         q=to_dev(q, "f32"), v=to_dev(v, "f32"))
    torch.cuda.synchronize()
    for name, g, r in zip(("du", "dq", "dv", "dk", "dD"), got, ref):
        r = r.cpu().numpy().astype(np.float64)
        err = rel_l2(g.reshape(-1), r.reshape(-1))
        say(f"   {name}: rel L2 {err:.3e}")
        assert err <= TOL["f32"], (name, err)


def test_partial_bwd_without_filter_gradient(lc):
    spec = wl.spec_partial(2, 2, 1000, 64, "bf16", gated=True, seed=43)
    d, dy, q, v = inputs(spec, "qv")
    du, dq, dv, dk, dD = run_pbwd(lc, d, dy, q, v, need_dk=False)
    assert dk is None and dD is None
    ref = run_pbwd(lc, d, dy, q, v)
    assert np.array_equal(du, ref[0]) and np.array_equal(dq, ref[1]) and np.array_equal(dv, ref[2])

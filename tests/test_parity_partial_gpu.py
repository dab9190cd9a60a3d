"""GPU parity of the partial convolution (filter of L taps, sequence of any length N):
lconv_fftconv_partial_fwd through the C ABI against the float64 short-filter oracle
(oracle.conv1d_short_points).

Tolerance as for the forward: max relative L2 error 1e-4 (fp32) and 2e-2 (bf16 / fp16) per
fully checked (b, h) row; pooled over the sampled positions of the long case.
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


def run_partial(lc, d, q, v):
    import torch
    dt = d["dtype"]
    L = d["k"].shape[1]
    kf = lc.filter_fft(to_dev(d["k"], dt))
    y = lc.fftconv_partial(to_dev(d["u"], dt), kf, to_dev(d["D"], dt), L, q=to_dev(q, dt), v=to_dev(v, dt))
    torch.cuda.synchronize()
    return from_dev(y, dt)


# (B, H, N, L, gates): N below, at and above L and the block length C = M/2, ragged block counts
CASES = [
    (1, 2, 64, 8, ""),
    (3, 2, 1000, 64, "qv"),
    (2, 3, 4096, 200, "q"),
    (4, 2, 520, 512, "v"),        # N barely above C = 512
    (2, 2, 512, 512, "qv"),       # N == L == C
    (3, 2, 256, 1000, "qv"),      # N < L
    (2, 2, 10000, 1000, "qv"),
    (5, 1, 24584, 2048, "qv"),    # 7 blocks (C = 4096), ragged last block
    (2, 2, 16384, 4096, "qv"),    # M = 8192 (one sequence per workgroup iteration)
    (1, 3, 12296, 4096, "v"),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("B,H,N,L,gates", CASES)
def test_partial_full_rows(lc, nthreads, dtype, B, H, N, L, gates):
    spec = wl.spec_partial(B, H, N, L, dtype, gated=True, seed=500 + N + L + B)
    say(f"[partial] dtype={dtype} B={B} H={H} N={N} L={L} gates={gates!r} seed={spec.seed}")
    d = wl.make(spec)
    q = d["q"] if "q" in gates else None
    v = d["v"] if "v" in gates else None
    y = run_partial(lc, d, q, v)
    assert np.all(np.isfinite(y))
    pts = [(b, h, t) for b in range(B) for h in range(H) for t in range(N)]
    ref = oracle.conv1d_short_points(d["u"], d["k"], d["D"], pts, q=q, v=v, dt=DT_ORACLE[dtype],
                                     nthreads=nthreads).reshape(B, H, N)
    err = float(rel_l2_rows(y, ref).max())
    say(f"   max rel L2 = {err:.3e} (tol {TOL[dtype]})")
    assert err <= TOL[dtype]


def test_partial_long_sequence_sampled(lc, nthreads):
    """A 2^21-long sequence with a 4096-tap filter (512 blocks per row), bf16, sampled."""
    spec = wl.WORKLOADS["partial_bf16_b1_h64_n2097152_l4096"]
    say(f"[partial long] {spec.name} seed={spec.seed}")
    d = wl.make(spec)
    y = run_partial(lc, d, d["q"], d["v"])
    pts = wl.sample_points_1d(spec.B, spec.H, spec.N, seed=2100)
    # block boundaries of the 4096-position blocks on a few rows
    extra = [(0, h, t) for h in (0, 63) for t in (4095, 4096, 4097, 8191, 8192, 2 ** 21 - 4096, 2 ** 21 - 1)]
    pts = np.concatenate([pts, np.asarray(extra, np.int64)], 0)
    ref = oracle.conv1d_short_points(d["u"], d["k"], d["D"], pts, q=d["q"], v=d["v"], dt=DT_ORACLE["bf16"],
                                     nthreads=nthreads)
    got = y[pts[:, 0], pts[:, 1], pts[:, 2]]
    assert np.all(np.isfinite(got))
    err = rel_l2(got, ref)
    say(f"   pooled rel L2 over {len(pts)} positions = {err:.3e}")
    assert err <= TOL["bf16"]


def test_partial_matches_full_length_call(lc):
    """With L = N the partial call computes the same convolution as the full-length call."""
    import torch
    spec = wl.spec_partial(3, 2, 2048, 2048, "bf16", gated=True, seed=31)
    say(f"[partial vs full] seed={spec.seed}")
    d = wl.make(spec)
    y_part = run_partial(lc, d, d["q"], d["v"])
    k = to_dev(d["k"], "bf16")
    y_full = lc.fftconv(to_dev(d["u"], "bf16"), lc.filter_fft(k), to_dev(d["D"], "bf16"),
                        q=to_dev(d["q"], "bf16"), v=to_dev(d["v"], "bf16"))
    torch.cuda.synchronize()
    err = float(rel_l2_rows(y_part, from_dev(y_full, "bf16")).max())
    say(f"   max rel L2 between the two paths = {err:.3e}")
    assert err <= TOL["bf16"]

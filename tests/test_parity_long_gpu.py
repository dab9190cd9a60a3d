"""GPU parity of the multi-pass path at every column length: transform lengths M = M1 x 8192 for
M1 = 32 .. 1024 (N from 131072 up to 2,300,000, the length of the longest human genes the
FlashFFTConv abstract mentions), against the float64 oracle at sampled positions.

Each case: 3584 uniform positions plus structured ones (t = 0, 1, N-2, N-1 and both sides of
power-of-two block boundaries, including the 8192-point rows of the split), pooled relative L2
error against oracle.conv1d_points; tolerance 2e-2 (bf16 / fp16), 1e-4 (fp32).
"""
import numpy as np
import pytest

import oracle
from fft_long_convolution_amd import workloads as wl
from tests.gpu_util import DT_ORACLE, TOL, from_dev, rel_l2, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lc():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fft_long_convolution_amd import lconv
    lconv.load()
    return lconv


# (B, H, N, dtype, gated): column lengths M1 = 32, 64, 128, 256, 256, 256, 512, 1024.  The 16-bit
# cases with M1 >= 256 run the matrix-core column passes (both batch rows of a pair, an odd
# batch's lone last row, and one-row sequences); fp32 keeps the vector-ALU ones.
CASES = [
    (2, 2, 131072, "bf16", True),
    (1, 3, 262144, "f16", False),
    (3, 1, 524288, "bf16", True),
    (1, 2, 1048576, "f32", False),
    (1, 2, 1000000, "bf16", True),      # not a power of two
    (3, 1, 600000, "f16", True),        # M1 = 256, odd batch
    (2, 1, 1572864, "f16", True),       # M1 = 512
    (1, 2, 2300000, "bf16", False),     # M = 2^23, M1 = 1024
    (1, 3, 1572864, "bf16", True),      # M1 = 512, one real row per sequence: paired inverse, odd count
    (1, 5, 2097152, "f16", False),      # M1 = 512, paired inverse, odd count
    (1, 3, 700000, "f16", True),        # M1 = 256, one real row per sequence, odd count
    (1, 3, 2200000, "bf16", True),      # M1 = 1024, one real row per sequence, odd count
]


@pytest.mark.parametrize("B,H,N,dtype,gated", CASES)
def test_long_sampled(lc, nthreads, B, H, N, dtype, gated):
    import torch
    spec = wl.spec_1d(B, H, N, dtype, gated=gated, seed=900 + N % 1000 + B, decay=1e-5)
    M = oracle.transform_length(N)
    say(f"[long] dtype={dtype} B={B} H={H} N={N} M={M} M1={M // 8192} gated={gated} seed={spec.seed}")
    d = wl.make(spec)
    k = to_dev(d["k"], dtype)
    u, q, v, D = (to_dev(d[x], dtype) for x in ("u", "q", "v", "D"))
    kf = lc.filter_fft(k)
    y = lc.fftconv(u, kf, D, q=q, v=v)
    torch.cuda.synchronize()
    got_all = from_dev(y, dtype)
    pts = wl.sample_points_1d(B, H, N, seed=2200 + N % 997)
    ref = oracle.conv1d_points(d["u"], d["k"], d["D"], pts, q=d["q"], v=d["v"], dt=DT_ORACLE[dtype],
                               nthreads=nthreads)
    got = got_all[pts[:, 0], pts[:, 1], pts[:, 2]]
    assert np.all(np.isfinite(got))
    err = rel_l2(got, ref)
    say(f"   pooled rel L2 over {len(pts)} positions = {err:.3e} (tol {TOL[dtype]})")
    assert err <= TOL[dtype]

"""GPU parity of the 2D gradients: lconv_fftconv2d_bwd through the C ABI against the float64
oracle (oracle.conv2d_bwd, pinned element by element in tests/test_oracle2d_bwd.py).

Tolerance as for the 2D forward (bf16 / fp16 inputs): max relative L2 2e-2 per image of du and
per channel of dk; dD as one vector over channels.  Any non-finite output fails.
"""
import numpy as np
import pytest

import oracle
from fft_long_convolution_amd import workloads as wl
from tests.gpu_util import DT_ORACLE, from_dev, rel_l2, rel_l2_rows, say, to_dev

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module")
def lc():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fft_long_convolution_amd import lconv
    lconv.load()
    return lconv


def run_bwd2d(lc, d, dy, need_dk=True):
    import torch
    dt = d["dtype"]
    u, k, D = (to_dev(d[x], dt) for x in ("u", "k", "D"))
    kf = lc.filter_fft2d(k)
    du, dk, dD = lc.fftconv2d_bwd(to_dev(dy, dt), u, kf, D, need_dk=need_dk)
    torch.cuda.synchronize()
    f32 = lambda t: None if t is None else t.cpu().numpy().astype(np.float64)
    return from_dev(du, dt), f32(dk), f32(dD)


def check(d, dy, got, images=None, chans=None):
    du, dk, dD = got
    spec = d["spec"]
    B, C = spec.B, spec.C
    images = images if images is not None else [(b, c) for b in range(B) for c in range(C)]
    chans = chans if chans is not None else list(range(C))
    r_du, r_dk, r_dD = oracle.conv2d_bwd(d["u"], d["k"], d["D"], dy, images=images, chans=chans,
                                         dt=DT_ORACLE[d["dtype"]])
    g_du = np.stack([du[b, c] for b, c in images])
    assert np.all(np.isfinite(g_du)) and np.all(np.isfinite(dk)) and np.all(np.isfinite(dD))
    n = len(images)
    errs = {"du": float(rel_l2_rows(g_du.reshape(n, -1), r_du.reshape(n, -1)).max()),
            "dk": float(rel_l2_rows(dk[chans].reshape(len(chans), -1), r_dk.reshape(len(chans), -1)).max()),
            "dD": rel_l2(dD[chans], r_dD)}
    return errs


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("Hs,Ws,B,C", [(128, 128, 3, 2), (16, 16, 2, 3), (128, 64, 2, 3), (37, 24, 3, 2),
                                       (1, 8, 3, 1), (127, 120, 1, 2), (100, 128, 4, 1)])
def test_2d_bwd_full(lc, dtype, Hs, Ws, B, C):
    """Every image of du and every channel of dk, dD against the oracle: square, rectangular and
    odd shapes, odd and even batches."""
    spec = wl.Conv2DSpec(f"t2db_{dtype}_{Hs}x{Ws}", B, C, Hs, dtype, seed=800 + Hs + Ws + B, Ws=Ws)
    say(f"[2d bwd] dtype={dtype} B={B} C={C} Hs={Hs} Ws={Ws} seed={spec.seed}")
    d = wl.make(spec)
    dy = wl.make_grad_2d(spec)
    errs = check(d, dy, run_bwd2d(lc, d, dy))
    say("   " + " ".join(f"{k}={e:.3e}" for k, e in errs.items()) + f" (tol {TOL})")
    for k, e in errs.items():
        assert e <= TOL, (k, e)


def test_2d_bwd_workload_sampled(lc):
    """The 2D workload (B8 C256 128 x 128, bf16): du on 24 images and dk, dD on 16 channels
    (first, last and seeded ones) against the oracle."""
    spec = wl.WORKLOADS["hyenand_2d_bf16_b8_c256_s128"]
    say(f"[2d bwd workload] {spec.name} seed={spec.seed}")
    d = wl.make(spec)
    dy = wl.make_grad_2d(spec)
    got = run_bwd2d(lc, d, dy)
    rng = np.random.default_rng(2500)
    images = [(0, 0), (spec.B - 1, spec.C - 1)] + [(int(b), int(c)) for b, c in
                                                  zip(rng.integers(0, spec.B, 22), rng.integers(0, spec.C, 22))]
    chans = sorted({0, spec.C - 1, *map(int, rng.integers(0, spec.C, 14))})
    errs = check(d, dy, got, images=images, chans=chans)
    say("   " + " ".join(f"{k}={e:.3e}" for k, e in errs.items()) + f" (tol {TOL})")
    for k, e in errs.items():
        assert e <= TOL, (k, e)


def test_2d_bwd_without_filter_gradient(lc):
    spec = wl.Conv2DSpec("t2db_nodk", 2, 2, 64, "bf16", seed=71, Ws=32)
    d = wl.make(spec)
    dy = wl.make_grad_2d(spec)
    du, dk, dD = run_bwd2d(lc, d, dy, need_dk=False)
    assert dk is None and dD is None
    ref = run_bwd2d(lc, d, dy)
    assert np.array_equal(du, ref[0])

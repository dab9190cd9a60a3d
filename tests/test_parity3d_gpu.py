"""GPU parity of the 3D (volume) convolution: lconv_filter_fft3d + lconv_fftconv3d_fwd through
the C ABI against the float64 direct-sum oracle (oracle.conv3d_points).

Tolerance as for 1D and 2D: max relative L2 error 1e-4 (fp32), 2e-2 (bf16 / fp16) per fully
checked volume; pooled over the sampled voxels where the oracle samples.
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


def run3d(lc, d):
    import torch
    dt = d["dtype"]
    kf = lc.filter_fft3d(to_dev(d["k"], dt))
    y = lc.fftconv3d(to_dev(d["u"], dt), kf, to_dev(d["D"], dt))
    torch.cuda.synchronize()
    return from_dev(y, dt)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("B", [1, 3, 4])
def test_3d_s16_full(lc, nthreads, dtype, B):
    C, S = 2, 16
    spec = wl.spec_3d(B, C, S, dtype, seed=40 + B)
    say(f"[3d] dtype={dtype} B={B} C={C} S={S} seed={spec.seed}")
    d = wl.make(spec)
    y = run3d(lc, d)
    assert np.all(np.isfinite(y))
    g = np.stack(np.meshgrid(np.arange(B), np.arange(C), np.arange(S), np.arange(S), np.arange(S),
                             indexing="ij"), -1).reshape(-1, 5)
    ref = oracle.conv3d_points(d["u"], d["k"], d["D"], g, dt=DT_ORACLE[dtype], nthreads=nthreads)
    err = float(rel_l2_rows(y.reshape(B * C, -1), ref.reshape(B * C, -1)).max())
    say(f"   max rel L2 per volume = {err:.3e} (tol {TOL[dtype]})")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("B", [1, 2])
def test_3d_s32_full(lc, nthreads, dtype, B):
    """S = 32 in 16-bit types (the matrix-core passes): every voxel of every volume, both images
    of a batch pair (B = 2) and a lone image (B = 1)."""
    C, S = 1, 32
    spec = wl.spec_3d(B, C, S, dtype, seed=90 + B)
    say(f"[3d] dtype={dtype} B={B} C={C} S={S} seed={spec.seed} (every voxel)")
    d = wl.make(spec)
    y = run3d(lc, d)
    assert np.all(np.isfinite(y))
    g = np.stack(np.meshgrid(np.arange(B), np.arange(C), np.arange(S), np.arange(S), np.arange(S),
                             indexing="ij"), -1).reshape(-1, 5)
    ref = oracle.conv3d_points(d["u"], d["k"], d["D"], g, dt=DT_ORACLE[dtype], nthreads=nthreads)
    err = float(rel_l2_rows(y.reshape(B * C, -1), ref.reshape(B * C, -1)).max())
    say(f"   max rel L2 per volume = {err:.3e} (tol {TOL[dtype]})")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_3d_s32_sampled(lc, nthreads, dtype):
    B, C, S = 3, 3, 32
    spec = wl.spec_3d(B, C, S, dtype, seed=77)
    say(f"[3d] dtype={dtype} B={B} C={C} S={S} seed={spec.seed}")
    d = wl.make(spec)
    y = run3d(lc, d)
    pts = wl.sample_points_3d(B, C, S, n=2048, seed=2301)
    ref = oracle.conv3d_points(d["u"], d["k"], d["D"], pts, dt=DT_ORACLE[dtype], nthreads=nthreads)
    got = y[pts[:, 0], pts[:, 1], pts[:, 2], pts[:, 3], pts[:, 4]]
    assert np.all(np.isfinite(got))
    err = rel_l2(got, ref)
    say(f"   pooled rel L2 over {len(pts)} voxels = {err:.3e} (tol {TOL[dtype]})")
    assert err <= TOL[dtype]


def test_3d_workload_sampled(lc, nthreads):
    spec = wl.WORKLOADS["hyenand_3d_bf16_b4_c128_s32"]
    say(f"[3d workload] {spec.name} seed={spec.seed}")
    d = wl.make(spec)
    y = run3d(lc, d)
    pts = wl.sample_points_3d(spec.B, spec.C, spec.S, n=2048, seed=2007)
    ref = oracle.conv3d_points(d["u"], d["k"], d["D"], pts, dt=DT_ORACLE["bf16"], nthreads=nthreads)
    got = y[pts[:, 0], pts[:, 1], pts[:, 2], pts[:, 3], pts[:, 4]]
    err = rel_l2(got, ref)
    say(f"   pooled rel L2 over {len(pts)} voxels = {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= TOL["bf16"]

"""GPU parity of the 2D path (centred full-size kernel, linear convolution cropped to the input
window, plus D skip) against the float64 CPU oracles: the naive separable-DFT oracle for whole
images and direct summation at sampled positions.  Tolerance: max relative L2 2e-2 per image
(bf16 / fp16 inputs), pooled over sampled positions at the full workload size."""
import numpy as np
import pytest

import oracle
from fft_long_convolution_amd import workloads as wl
from tests.gpu_util import DT_ORACLE, from_dev, rel_l2, rel_l2_rows, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lc():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fft_long_convolution_amd import lconv
    lconv.load()
    return lconv


def run_2d(lc, d):
    import torch
    dt = d["dtype"]
    u, k, D = (to_dev(d[x], dt) for x in ("u", "k", "D"))
    kf = lc.filter_fft2d(k)
    y = lc.fftconv2d(u, kf, D)
    torch.cuda.synchronize()
    return from_dev(y, dt)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("B,C", [(3, 2), (2, 5), (1, 1)])
def test_2d_full_images(lc, dtype, B, C):
    spec = wl.Conv2DSpec(f"t2d_{dtype}_{B}_{C}", B, C, 128, dtype, seed=50 + B * 7 + C)
    say(f"[2d] dtype={dtype} B={B} C={C} seed={spec.seed}")
    d = wl.make(spec)
    y = run_2d(lc, d)
    assert np.all(np.isfinite(y))
    imgs = [(b, c) for b in range(B) for c in range(C)]
    ref = oracle.conv2d_dft(d["u"], d["k"], d["D"], imgs, dt=DT_ORACLE[dtype]).reshape(B, C, -1)
    err = rel_l2_rows(y.reshape(B, C, -1), ref).max()
    say(f"   max rel L2 = {err:.3e}")
    assert err <= 2e-2


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("Hs,Ws,B,C", [(128, 64, 2, 3), (100, 128, 3, 2), (37, 24, 2, 2), (1, 8, 3, 1),
                                       (64, 128, 1, 4), (127, 120, 2, 1)])
def test_2d_rectangular_full_images(lc, dtype, Hs, Ws, B, C):
    """Hs x Ws images, sides up to 128 (odd rows included): every image against the naive-DFT
    oracle with the centre tap at (Hs // 2, Ws // 2)."""
    spec = wl.Conv2DSpec(f"t2d_{dtype}_{Hs}x{Ws}", B, C, Hs, dtype, seed=600 + Hs + Ws, Ws=Ws)
    say(f"[2d rect] dtype={dtype} B={B} C={C} Hs={Hs} Ws={Ws} seed={spec.seed}")
    d = wl.make(spec)
    y = run_2d(lc, d)
    assert y.shape == (B, C, Hs, Ws) and np.all(np.isfinite(y))
    imgs = [(b, c) for b in range(B) for c in range(C)]
    ref = oracle.conv2d_dft(d["u"], d["k"], d["D"], imgs, dt=DT_ORACLE[dtype]).reshape(B, C, -1)
    err = rel_l2_rows(y.reshape(B, C, -1), ref).max()
    say(f"   max rel L2 = {err:.3e}")
    assert err <= 2e-2


def test_2d_delta_kernel_is_identity(lc):
    """Centre tap 1 and D = 0: the output reproduces the input (up to bf16 rounding)."""
    spec = wl.Conv2DSpec("delta2d", 2, 3, 128, "bf16", seed=9)
    d = wl.make(spec)
    k = np.zeros((3, 128, 128), np.float32)
    k[:, 64, 64] = 1
    d["k"] = wl.to_storage(k, "bf16")
    d["D"] = wl.to_storage(np.zeros(3, np.float32), "bf16")
    say("[2d] delta kernel")
    y = run_2d(lc, d)
    u = wl.storage_to_f64(d["u"], "bf16")
    assert rel_l2(y, u) <= 1e-2


def test_2d_workload_hyenand(lc, nthreads):
    """B8 C256 128x128: every one of the 2,048 images against the naive-DFT oracle, plus 4096
    sampled positions by direct summation."""
    name = "hyenand_2d_bf16_b8_c256_s128"
    d = wl.make(name)
    say(f"[workload] {name}")
    y = run_2d(lc, d)
    assert np.all(np.isfinite(y))
    pts = wl.sample_points_2d(8, 256, 128, seed=2005)
    refp = oracle.conv2d_points(d["u"], d["k"], d["D"], pts, dt=oracle.DT_BF16, nthreads=nthreads)
    err = rel_l2(y[pts[:, 0], pts[:, 1], pts[:, 2], pts[:, 3]], refp)
    worst, worst_at, max_abs = 0.0, None, 0.0
    for c0 in range(0, 256, 32):   # 32 channels (256 images) at a time bounds the oracle's memory
        imgs = [(b, c) for c in range(c0, c0 + 32) for b in range(8)]
        ref = oracle.conv2d_dft(d["u"], d["k"], d["D"], imgs, dt=oracle.DT_BF16)
        got = np.stack([y[b, c] for b, c in imgs])
        e = rel_l2_rows(got.reshape(len(imgs), -1), ref.reshape(len(imgs), -1))
        i = int(np.argmax(e))
        if e[i] > worst:
            worst, worst_at = float(e[i]), imgs[i]
        max_abs = max(max_abs, float(np.max(np.abs(got - ref))))
    say(f"   all 2048 images: max rel L2 = {worst:.3e} at (b,c)={worst_at}, max abs err {max_abs:.3e}; "
        f"sampled pooled rel L2 = {err:.3e}")
    assert err <= 2e-2 and worst <= 2e-2


def test_2d_more_items_than_workgroups(lc):
    """300 channels of one batch pair on at most 256 workgroups: workgroups renumbered XCD by XCD,
    some taking a second item.  Full images of channels on both sides of the first round."""
    B, C = 2, 300
    spec = wl.Conv2DSpec("t2d_bf16_2_300", B, C, 128, "bf16", seed=77)
    say(f"[2d] B={B} C={C} seed={spec.seed}")
    d = wl.make(spec)
    y = run_2d(lc, d)
    chans = [0, 1, 7, 8, 31, 32, 255, 256, 257, 299]
    imgs = [(b, c) for b in range(B) for c in chans]
    ref = oracle.conv2d_dft(d["u"], d["k"], d["D"], imgs, dt=DT_ORACLE["bf16"]).reshape(len(imgs), -1)
    got = np.stack([y[b, c].reshape(-1) for b, c in imgs])
    err = rel_l2_rows(got, ref).max()
    say(f"   max rel L2 = {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= 2e-2

"""Run-to-run bitwise determinism of every GPU path: the same call on the same inputs twice must
give identical bits (no atomics, no order-dependent sums; a race in LDS or a missing barrier
would show up as a difference).  One case per path: the multi-pass forward, the 2D and 3D
convolutions, the gradients of one workgroup per transform and of the multi-pass path, the
state-space, partial and frequency-sparse calls."""
import numpy as np
import pytest

from fft_long_convolution_amd import workloads as wl
from tests.gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lc():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fft_long_convolution_amd import lconv
    lconv.load()
    return lconv


def same(a, b):
    import torch
    if a is None or b is None:
        return a is None and b is None
    if a.dtype in (torch.bfloat16, torch.float16):
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def twice(fn):
    import torch
    r1 = fn()
    torch.cuda.synchronize()
    r2 = fn()
    torch.cuda.synchronize()
    r1 = r1 if isinstance(r1, tuple) else (r1,)
    r2 = r2 if isinstance(r2, tuple) else (r2,)
    return all(same(a, b) for a, b in zip(r1, r2))


def dev1d(spec):
    d = wl.make(spec)
    dt = spec.dtype
    return d, tuple(to_dev(d[x], dt) for x in ("u", "q", "v", "k", "D"))


def test_multipass_forward(lc):
    spec = wl.spec_1d(3, 2, 65536, "bf16", gated=True, seed=901, decay=1e-4)
    say(f"[determinism] multi-pass forward B3 H2 N65536 seed={spec.seed}")
    d, (u, q, v, k, D) = dev1d(spec)
    kf = lc.filter_fft(k)
    assert twice(lambda: lc.fftconv(u, kf, D, q=q, v=v))
    assert twice(lambda: lc.filter_fft(k))


@pytest.mark.parametrize("N", [4096, 16384])
def test_gradients(lc, N):
    spec = wl.spec_1d(3, 2, N, "bf16", gated=True, seed=902 + N, decay=1e-4)
    say(f"[determinism] gradients B3 H2 N{N} seed={spec.seed}")
    d, (u, q, v, k, D) = dev1d(spec)
    kf = lc.filter_fft(k)
    dy = to_dev(wl.make_grad_1d(spec), "bf16")
    assert twice(lambda: lc.fftconv_bwd(dy, u, kf, D, q=q, v=v))


def test_2d_and_3d(lc):
    say("[determinism] 2D B3 C2 128x128 and 3D B2 C2 16^3")
    d = wl.make(wl.Conv2DSpec("det2d", 3, 2, 128, "bf16", seed=903))
    u, k, D = (to_dev(d[x], "bf16") for x in ("u", "k", "D"))
    kf = lc.filter_fft2d(k)
    assert twice(lambda: lc.fftconv2d(u, kf, D))
    d3 = wl.make(wl.spec_3d(2, 2, 16, "bf16", seed=904))
    u3, k3, D3 = (to_dev(d3[x], "bf16") for x in ("u", "k", "D"))
    kf3 = lc.filter_fft3d(k3)
    assert twice(lambda: lc.fftconv3d(u3, kf3, D3))


def test_state_space_partial_sparse(lc):
    import torch
    say("[determinism] state-space, partial, frequency-sparse")
    spec = wl.spec_1d(2, 2, 8192, "bf16", gated=True, seed=905)
    d, (u, q, v, k, D) = dev1d(spec)
    lam, W = wl.ssm_modes(2, 16, seed=906)
    prep = lc.ssm_prepare(torch.from_numpy(lam.astype(np.complex64)).cuda(),
                          torch.from_numpy(W.astype(np.complex64)).cuda(), 1024, torch.bfloat16)
    assert twice(lambda: lc.fftconv_ssm(u, prep, D, 16, 1024, q=q, v=v))
    kl = lc.filter_fft(k[:, :512].contiguous())
    assert twice(lambda: lc.fftconv_partial(u, kl, D, 512, q=q, v=v))
    s2 = wl.spec_1d(4, 3, 4096, "bf16", gated=True, seed=907)
    d2, (u2, q2, v2, k2, D2) = dev1d(s2)
    kf2 = lc.filter_fft(k2)
    assert twice(lambda: lc.fftconv_sparse(u2, kf2, D2, [0, 1, 31, 5, 27], q=q2, v=v2))

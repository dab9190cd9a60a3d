"""Host-side checks of the torch wrappers (no GPU needed): every operand's dtype, shape and dense
layout, the opaque buffers' sizes, and the device, rejected before any call into the library."""
import pytest

torch = pytest.importorskip("torch")

from fft_long_convolution_amd import lconv  # noqa: E402


def gated(B=2, H=3, N=64, dt=torch.bfloat16):
    u = torch.zeros(B, H, N, dtype=dt)
    q, v = torch.zeros_like(u), torch.zeros_like(u)
    D = torch.zeros(H, dtype=dt)
    kf = torch.zeros(lconv.lconv_filter_fft_bytes(H, N, lconv.dtype_code(dt)), dtype=torch.uint8)
    return u, kf, D, q, v


def raises(match, fn, *a, **kw):
    with pytest.raises((ValueError, TypeError), match=match):
        fn(*a, **kw)


def test_fftconv_rejects_noncontiguous_views():
    u, kf, D, q, v = gated()
    ut = torch.zeros(2, 64, 3, dtype=torch.bfloat16).transpose(1, 2)    # [2, 3, 64], strided
    raises("contiguous", lconv.fftconv, ut, kf, D)
    raises("contiguous", lconv.fftconv, u, kf, D, q=torch.zeros(2, 64, 3, dtype=torch.bfloat16).transpose(1, 2))
    raises("contiguous", lconv.fftconv, u, kf, torch.zeros(6, dtype=torch.bfloat16)[::2])


def test_fftconv_rejects_dtype_and_shape_mismatches():
    u, kf, D, q, v = gated()
    raises("dtype", lconv.fftconv, u, kf, D, q=q.half())
    raises("dtype", lconv.fftconv, u, kf, D, v=v.float())
    raises("dtype", lconv.fftconv, u, kf, D.float())
    raises("shape", lconv.fftconv, u, kf, torch.zeros(4, dtype=torch.bfloat16))
    raises("shape", lconv.fftconv, u, kf, D, q=torch.zeros(2, 3, 32, dtype=torch.bfloat16))
    raises("shape", lconv.fftconv, u, kf, D, out=torch.zeros(1, 3, 64, dtype=torch.bfloat16))
    raises("dtype", lconv.fftconv, u.to(torch.float64), kf, D)
    raises("3-D", lconv.fftconv, u[0], kf, D)


def test_fftconv_rejects_a_spectrum_of_another_shape_or_dtype():
    u, kf, D, q, v = gated(N=64)
    other_n = torch.zeros(lconv.lconv_filter_fft_bytes(3, 4096, lconv.BF16), dtype=torch.uint8)
    raises("made for another shape", lconv.fftconv, u, other_n, D)
    other_h = torch.zeros(lconv.lconv_filter_fft_bytes(2, 64, lconv.BF16), dtype=torch.uint8)
    raises("made for another shape", lconv.fftconv, u, other_h, D)
    raises("uint8", lconv.fftconv, u, kf.float(), D)


def test_fftconv_rejects_host_tensors():
    u, kf, D, q, v = gated()
    raises("GPU tensor", lconv.fftconv, u, kf, D, q=q, v=v)


def test_gradient_and_training_pair_checks():
    u, kf, D, q, v = gated()
    dy = torch.zeros_like(u)
    raises("dtype", lconv.fftconv_bwd, dy.half(), u, kf, D, q=q, v=v)
    raises("shape", lconv.fftconv_bwd, dy, u, kf, D, q=q, v=v, c=torch.zeros(2, 3, 8, dtype=torch.bfloat16))
    raises("dtype", lconv.fftconv_bwd, dy, u, kf, D, q=q, v=v, c=torch.zeros(2, 3, 64, dtype=torch.float16))
    raises("required", lconv.fftconv_bwd, None, u, kf, D)
    raises("contiguous", lconv.fftconv_save, u, kf, D,
           q=torch.zeros(2, 64, 3, dtype=torch.bfloat16).transpose(1, 2))
    raises("GPU tensor", lconv.fftconv_bwd, dy, u, kf, D, q=q, v=v)


def test_partial_and_sparse_checks():
    u, kf, D, q, v = gated(N=4096)
    kf_l = torch.zeros(lconv.lconv_filter_fft_bytes(3, 16, lconv.BF16), dtype=torch.uint8)
    raises("made for another shape", lconv.fftconv_partial, u, kf, D, 16)   # spectrum of N taps, not L
    raises("GPU tensor", lconv.fftconv_partial, u, kf_l, D, 16)
    raises("dtype", lconv.fftconv_sparse, u, kf, D, [0], q=q.float())


def test_filter_fft_checks():
    raises("contiguous", lconv.filter_fft, torch.zeros(64, 3, dtype=torch.bfloat16).t())
    raises("2-D", lconv.filter_fft, torch.zeros(3, dtype=torch.bfloat16))
    raises("GPU tensor", lconv.filter_fft, torch.zeros(3, 64, dtype=torch.bfloat16))


def test_2d_checks():
    u = torch.zeros(2, 3, 128, 64, dtype=torch.bfloat16)
    D = torch.zeros(3, dtype=torch.bfloat16)
    kf = torch.zeros(lconv.lconv_filter_fft2d_bytes(3, 128, 64, lconv.BF16), dtype=torch.uint8)
    raises("contiguous", lconv.fftconv2d, torch.zeros(2, 3, 64, 128, dtype=torch.bfloat16).transpose(2, 3), kf, D)
    raises("shape", lconv.fftconv2d, u, kf, torch.zeros(2, dtype=torch.bfloat16))
    raises("made for another shape", lconv.fftconv2d, u, kf[:100], D)
    raises("GPU tensor", lconv.fftconv2d, u, kf, D)
    raises("contiguous", lconv.filter_fft2d, torch.zeros(3, 64, 128, dtype=torch.bfloat16).transpose(1, 2))


def test_3d_and_state_space_checks():
    u = torch.zeros(1, 2, 16, 16, 16, dtype=torch.bfloat16)
    D = torch.zeros(2, dtype=torch.bfloat16)
    kf = torch.zeros(lconv.lconv_filter_fft3d_bytes(2, 16, lconv.BF16), dtype=torch.uint8)
    raises("expected", lconv.fftconv3d, torch.zeros(1, 2, 16, 16, 8, dtype=torch.bfloat16), kf, D)
    raises("made for another shape", lconv.fftconv3d, u, kf[:-16], D)
    raises("GPU tensor", lconv.fftconv3d, u, kf, D)
    lam = torch.zeros(2, 4, dtype=torch.complex64)
    raises("dtype", lconv.ssm_prepare, lam, torch.zeros(2, 4, dtype=torch.complex128), 256, torch.bfloat16)
    raises("shape", lconv.ssm_prepare, lam, torch.zeros(2, 5, dtype=torch.complex64), 256, torch.bfloat16)
    raises("GPU tensor", lconv.ssm_prepare, lam, lam.clone(), 256, torch.bfloat16)

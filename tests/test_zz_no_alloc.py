"""The allocation-free forward call (lconv_fftconv_fwd_noalloc, workspace from the library's static
scratch buffer) against the ordinary forward call (lconv_fftconv_fwd, caller-owned workspace),
both through the C ABI.  The two run the same kernels on the same inputs, so the outputs must be
bit-equal.  The calls run in a row, each later one on a smaller input than the one before, so
the scratch buffer still holds the previous call's contents when the next one starts."""
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


def _noalloc(lc, u, kf, D, y, q, v, B, H, N, dtc):
    import torch
    p = lambda t: None if t is None else t.data_ptr()
    return lc.lconv_fftconv_fwd_noalloc(u.data_ptr(), kf.data_ptr(), D.data_ptr(), y.data_ptr(), p(q), p(v),
                                        B, H, N, dtc, torch.cuda.current_stream().cuda_stream)


# (B, H, N, dtype, gated), largest first
SEQUENCE = [
    (2, 10, 2 ** 20, "bf16", True),   # multi-pass: 10 transforms of 8 MiB, two chunks of the buffer
    (3, 2, 65536, "f32", False),      # multi-pass, fp32 transforms
    (1, 3, 5000, "bf16", True),       # N not a multiple of 8: staged rows, then multi-pass
    (3, 4, 4096, "f16", True),        # single pass: no scratch used
]


def test_noalloc_matches_forward_twice_shrinking(lc):
    import torch
    for (B, H, N, dt, gated) in SEQUENCE:
        spec = wl.spec_1d(B, H, N, dt, gated=gated, seed=4100 + N + B)
        say(f"[noalloc] dtype={dt} B={B} H={H} N={N} gated={gated} seed={spec.seed}")
        d = wl.make(spec)
        k = to_dev(d["k"], dt)
        u, q, v, D = (to_dev(d[x], dt) for x in ("u", "q", "v", "D"))
        dtc = lc.dtype_code(u.dtype)
        assert lc.lconv_prepare(N, dtc) == 0
        kf = lc.filter_fft(k)
        y_ref = lc.fftconv(u, kf, D, q=q, v=v)
        y = torch.full_like(u, float("nan"))
        st = _noalloc(lc, u, kf, D, y, q, v, B, H, N, dtc)
        assert st == 0, lc.status_string(st)
        torch.cuda.synchronize()
        assert torch.isfinite(y.float()).all()
        same = torch.equal(y.view(torch.int16) if y.element_size() == 2 else y.view(torch.int32),
                           y_ref.view(torch.int16) if y.element_size() == 2 else y_ref.view(torch.int32))
        say(f"   bit-equal to lconv_fftconv_fwd: {same}")
        assert same


def test_noalloc_rejects_beyond_the_buffer(lc):
    """A call whose staging alone fills the buffer is refused on the host, before any launch."""
    assert lc.lconv_prepare(4096, lc.F32) == 0        # sets up this device's buffer
    A, Bq, C, Y = (0x100000000 * (i + 1) for i in range(4))  # never dereferenced
    N = 2 ** 22 - 1                                   # staged: 4 x 2^22 fp32 = 64 MiB
    st = lc.lconv_fftconv_fwd_noalloc(A, Bq, C, Y, None, None, 1, 1, N, lc.F32, None)
    assert st == 9, lc.status_string(st)              # LCONV_ERR_SCRATCH_LIMIT

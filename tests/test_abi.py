"""C-ABI tests that need no GPU: the library loads, exports every declared symbol, answers
size queries, and rejects bad arguments with the documented status before any HIP call."""
import ctypes

import pytest

from fft_long_convolution_amd import lconv

F32, F16, BF16 = lconv.F32, lconv.F16, lconv.BF16
OK, NULLP, SHAPE, UNSUP, MISAL, ALIAS, WSERR, HIPERR = range(8)

# fake, 16-byte aligned "device" addresses: validation must reject before touching them
A, Bq, C, Dd, Y, W = (0x100000 * (i + 1) for i in range(6))


@pytest.fixture(scope="module")
def lib():
    return lconv.load()


def test_exports_every_header_symbol(lib):
    names = lconv.header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
        assert callable(getattr(lconv, n)), n


def test_abi_version_and_strings(lib):
    assert lconv.lconv_abi_version() == 3
    for s in range(8):
        assert lconv.status_string(s)
    assert "unknown" in lconv.status_string(99)


def test_size_queries():
    # N=4096 -> M=8192 complex per channel
    assert lconv.lconv_filter_fft_bytes(768, 4096, BF16) == 768 * 8192 * 4
    assert lconv.lconv_filter_fft_bytes(4, 1024, F32) == 4 * 2048 * 8
    assert lconv.lconv_filter_fft_bytes(1, 8, F16) == 512 * 4           # minimum transform 512
    assert lconv.lconv_fftconv_workspace_bytes(16, 768, 4096, BF16) == 0  # single pass
    assert lconv.lconv_fftconv_workspace_bytes(4, 256, 65536, F16) > 0    # multi-pass
    assert lconv.lconv_filter_fft_workspace_bytes(64, 2 ** 21, BF16) > 0
    assert lconv.lconv_filter_fft_bytes(1, 12, BF16) == 512 * 4           # any N (ragged rows staged)
    assert lconv.lconv_fftconv_workspace_bytes(2, 3, 12, BF16) == 4 * 256  # 4 staged [6][16] tensors
    assert lconv.lconv_fftconv_workspace_bytes(2, 3, 16, BF16) == 0
    assert lconv.lconv_filter_fft_workspace_bytes(3, 12, BF16) == 256
    assert lconv.lconv_filter_fft_bytes(1, 2 ** 22 + 8, BF16) == 0        # too long
    assert lconv.lconv_filter_fft_bytes(1, 2300000, BF16) == 2 ** 23 * 4   # 2.3M: M = 2^23
    assert lconv.lconv_filter_fft_bytes(1, 8, 7) == 0                     # bad dtype
    assert lconv.lconv_filter_fft2d_bytes(256, 128, BF16) == 256 * 256 * 256 * 4
    assert lconv.lconv_filter_fft2d_bytes(1, 64, BF16) == 0


def fwd(u=A, kf=Bq, D=C, y=Y, q=None, v=None, B=2, H=3, N=64, dt=BF16, ws=None, wsb=0):
    return lconv.lconv_fftconv_fwd(u, kf, D, y, q, v, B, H, N, dt, ws, wsb, None)


def test_fwd_validation_errors():
    assert fwd(dt=5) == UNSUP
    assert fwd(B=-1) == SHAPE
    assert fwd(N=-8) == SHAPE
    assert fwd(B=2 ** 40, H=2 ** 20, N=2 ** 10) == SHAPE                 # overflow
    assert fwd(N=12) == WSERR                                              # ragged: staging space
    assert fwd(N=2 ** 22 + 8) == UNSUP
    assert fwd(u=None) == NULLP
    assert fwd(kf=None) == NULLP
    assert fwd(D=None) == NULLP
    assert fwd(y=None) == NULLP
    assert fwd(u=A + 2) == MISAL
    assert fwd(q=Bq + 8 + 0x1000) == MISAL
    assert fwd(y=A) == ALIAS                                               # y == u
    assert fwd(y=A + 16) == ALIAS                                          # overlap
    assert fwd(q=Y) == ALIAS
    assert fwd(N=65536, B=4, H=4) == WSERR                                 # multi-pass, no ws
    need = lconv.lconv_fftconv_workspace_bytes(4, 4, 65536, BF16)
    assert fwd(N=65536, B=4, H=4, ws=W + 0x10000000, wsb=need - 1) == WSERR


def test_empty_is_noop():
    assert fwd(B=0) == OK
    assert fwd(H=0) == OK
    assert fwd(N=0) == OK
    assert fwd(B=0, u=None, y=None) == OK
    assert lconv.lconv_filter_fft(None, None, 0, 64, BF16, None, 0, None) == OK
    assert lconv.lconv_fftconv2d_fwd(None, None, None, None, 0, 4, 128, BF16, None) == OK


def test_filter_fft_validation_errors():
    f = lconv.lconv_filter_fft
    assert f(A, Y, 3, 64, 9, None, 0, None) == UNSUP
    assert f(A, Y, -1, 64, BF16, None, 0, None) == SHAPE
    assert f(None, Y, 3, 64, BF16, None, 0, None) == NULLP
    assert f(A, None, 3, 64, BF16, None, 0, None) == NULLP
    assert f(A + 4, Y, 3, 64, BF16, None, 0, None) == MISAL
    assert f(A, A, 3, 64, BF16, None, 0, None) == ALIAS
    far = 1 << 40  # k_f far from k so only the missing workspace is wrong
    assert f(A, far, 3, 2 ** 21, BF16, None, 0, None) == WSERR


def test_2d_validation_errors():
    f = lconv.lconv_fftconv2d_fwd
    assert f(A, Bq, C, Y, 2, 3, 64, BF16, None) == UNSUP
    assert f(A, Bq, C, Y, 2, 3, 128, F32, None) == UNSUP
    assert f(None, Bq, C, Y, 2, 3, 128, BF16, None) == NULLP
    assert f(A + 2, Bq, C, Y, 2, 3, 128, BF16, None) == MISAL
    assert f(A, Bq, C, A, 2, 3, 128, BF16, None) == ALIAS
    assert f(A, Bq, C, Y, -2, 3, 128, BF16, None) == SHAPE


def test_no_device_gives_hip_error():
    """Valid arguments reach the HIP runtime; without a GPU that is LCONV_ERR_HIP."""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert fwd() == HIPERR


# more fake addresses for the gradient call (1 MiB apart, far larger than the test shapes)
G = [0x10000000 + 0x100000 * i for i in range(12)]


def bwd(dy=G[0], u=G[1], kf=G[2], D=G[3], q=None, v=None, du=G[4], dq=None, dv=None, dk=None,
        dD=None, B=2, H=3, N=64, dt=BF16):
    return lconv.lconv_fftconv_bwd(dy, u, kf, D, q, v, du, dq, dv, dk, dD, B, H, N, dt, None)


def test_bwd_validation_errors():
    assert bwd(dt=5) == UNSUP
    assert bwd(B=-1) == SHAPE
    assert bwd(H=2 ** 40, N=2 ** 30) == SHAPE                           # overflow
    assert bwd(N=12) == UNSUP
    assert bwd(N=8192) == UNSUP                                            # beyond one workgroup
    assert bwd(dy=None) == NULLP
    assert bwd(u=None) == NULLP
    assert bwd(kf=None) == NULLP
    assert bwd(D=None) == NULLP
    assert bwd(du=None) == NULLP
    assert bwd(q=G[5]) == NULLP                                            # q without dq
    assert bwd(v=G[6]) == NULLP                                            # v without dv
    assert bwd(dk=G[7] + 4) == MISAL
    assert bwd(q=G[5], dq=G[8] + 8) == MISAL
    assert bwd(du=G[0]) == ALIAS                                           # du == dy
    assert bwd(q=G[5], dq=G[4] + 16) == ALIAS                              # dq overlaps du
    assert bwd(dk=G[3]) == ALIAS                                           # dk overlaps D
    assert bwd(v=G[6], dv=G[2]) == ALIAS                                   # dv overlaps k_f
    assert bwd(dk=G[7], dD=G[7] + 16) == ALIAS                             # dD inside dk


def test_bwd_empty_and_ignored_outputs():
    assert bwd(H=0) == OK
    assert bwd(N=0) == OK
    assert bwd(B=0) == OK                                                  # nothing to zero
    assert bwd(B=0, dy=None, u=None, du=None) == OK
    # dq / dv without their gates are ignored: validation passes, and with no device the
    # call fails only at the first HIP call
    import torch
    if not torch.cuda.is_available():
        assert bwd(dq=G[0]) == HIPERR


def fsave(u=G[0], kf=G[1], D=G[2], y=G[3], c=G[4], q=None, v=None, B=2, H=3, N=64, dt=BF16):
    return lconv.lconv_fftconv_fwd_save(u, kf, D, y, c, q, v, B, H, N, dt, None)


def bsaved(dy=G[0], u=G[1], kf=G[2], D=G[3], q=None, v=None, c=None, du=G[4], dq=None, dv=None,
           dk=None, dD=None, B=2, H=3, N=64, dt=BF16):
    return lconv.lconv_fftconv_bwd_saved(dy, u, kf, D, q, v, c, du, dq, dv, dk, dD, B, H, N, dt, None)


def test_forward_save_validation_errors():
    assert fsave(dt=5) == UNSUP
    assert fsave(B=-1) == SHAPE
    assert fsave(N=12) == UNSUP                                            # N % 8
    assert fsave(N=8192) == UNSUP                                          # single transform only
    assert fsave(c=None) == NULLP
    assert fsave(y=None) == NULLP
    assert fsave(c=G[4] + 8) == MISAL
    assert fsave(c=G[3]) == ALIAS                                          # c == y
    assert fsave(c=G[0] + 64) == ALIAS                                     # c overlaps u
    assert fsave(v=G[5], y=G[5] + 32) == ALIAS                             # y overlaps v
    assert fsave(B=0) == OK and fsave(H=0) == OK and fsave(N=0) == OK


def test_saved_gradient_validation_errors():
    assert bsaved(v=G[6], dv=G[7]) == NULLP                                # v without c
    assert bsaved(v=G[6], dv=G[7], c=G[8] + 4) == MISAL
    assert bsaved(v=G[6], dv=G[7], c=G[4]) == ALIAS                        # du overlaps c
    assert bsaved(v=G[6], dv=G[8], c=G[8]) == ALIAS                        # dv == c
    assert bsaved(N=8192) == UNSUP
    assert bsaved(B=0) == OK
    import torch
    if not torch.cuda.is_available():                                      # c ignored without v
        assert bsaved(c=None) == HIPERR


def part(u=G[0], kf=G[1], D=G[2], y=G[3], q=None, v=None, B=2, H=3, N=64, L=32, dt=BF16):
    return lconv.lconv_fftconv_partial_fwd(u, kf, D, y, q, v, B, H, N, L, dt, None)


def test_partial_validation_errors():
    assert part(dt=5) == UNSUP
    assert part(B=-1) == SHAPE
    assert part(L=-8) == SHAPE
    assert part(L=12) == UNSUP                                            # L % 8
    assert part(L=8192) == UNSUP                                          # beyond one transform
    assert part(L=0) == UNSUP
    assert part(N=12) == UNSUP                                            # N % 8
    assert part(N=2 ** 41) == UNSUP
    assert part(B=2 ** 20, H=2 ** 10, N=2 ** 20, L=8) == UNSUP            # too many blocks
    assert part(u=None) == NULLP
    assert part(kf=None) == NULLP
    assert part(y=None) == NULLP
    assert part(D=G[2] + 4) == MISAL
    assert part(y=G[0]) == ALIAS
    assert part(q=G[3] + 16) == ALIAS


def test_partial_empty_is_noop():
    assert part(B=0) == OK
    assert part(H=0) == OK
    assert part(N=0) == OK


def sparse(u=G[0], kf=G[1], D=G[2], y=G[3], q=None, v=None, B=2, H=3, N=1000, keep=0b10000011, dt=BF16):
    return lconv.lconv_fftconv_sparse_fwd(u, kf, D, y, q, v, B, H, N, keep, dt, None)


def test_sparse_blocks_and_validation():
    assert lconv.lconv_freq_blocks(64) == 2          # M = 512
    assert lconv.lconv_freq_blocks(1000) == 8        # M = 2048
    assert lconv.lconv_freq_blocks(4096) == 32       # M = 8192
    assert lconv.lconv_freq_blocks(8192) == 0        # beyond one transform
    assert lconv.lconv_freq_blocks(12) == 0
    assert sparse(dt=5) == UNSUP
    assert sparse(B=-1) == SHAPE
    assert sparse(N=8192) == UNSUP
    assert sparse(keep=0b110) == UNSUP               # R = 8: mirror of 1 is 7, not 2
    assert sparse(keep=1 << 8) == UNSUP              # beyond R
    assert sparse(u=None) == NULLP
    assert sparse(D=G[2] + 2) == MISAL
    assert sparse(y=G[0]) == ALIAS
    assert sparse(B=0) == OK
    import torch
    if not torch.cuda.is_available():
        assert sparse(keep=0) == HIPERR               # valid (nothing kept): fails only at HIP
        assert sparse(N=4096, keep=0xffffffff) == HIPERR


def test_3d_sizes_and_validation():
    assert lconv.lconv_filter_fft3d_bytes(4, 32, BF16) == 4 * 64 ** 3 * 4
    assert lconv.lconv_filter_fft3d_bytes(4, 16, F32) == 4 * 32 ** 3 * 8
    assert lconv.lconv_filter_fft3d_bytes(4, 24, BF16) == 0                # S must be 16 or 32
    assert lconv.lconv_fftconv3d_workspace_bytes(4, 128, 32, BF16) > 0
    assert lconv.lconv_filter_fft3d_workspace_bytes(128, 32, BF16) > 0
    f3 = lambda u=G[0], kf=G[1], D=G[2], y=G[3], B=2, C=3, S=16, dt=BF16, ws=G[4], wsb=1 << 30: \
        lconv.lconv_fftconv3d_fwd(u, kf, D, y, B, C, S, dt, ws, wsb, None)
    assert f3(dt=5) == UNSUP
    assert f3(S=24) == UNSUP
    assert f3(B=-1) == SHAPE
    assert f3(u=None) == NULLP
    assert f3(D=G[2] + 2) == MISAL
    assert f3(y=G[0]) == ALIAS
    assert f3(ws=None) == WSERR
    assert f3(wsb=16) == WSERR
    assert f3(B=0) == OK


def test_ssm_sizes_and_validation():
    assert lconv.lconv_ssm_prep_bytes(64, 64, 4096, BF16) > 0
    assert lconv.lconv_ssm_prep_bytes(64, 64, 3000, BF16) == 0            # T a power of two
    assert lconv.lconv_ssm_prep_bytes(64, 300, 4096, BF16) == 0           # NS <= 256
    assert lconv.lconv_ssm_prep_bytes(64, 64, 8192, BF16) == 0
    # chunk sums and states (64 rows x 512 chunks x 64 modes), plus 64 scan parts per row
    assert lconv.lconv_fftconv_ssm_workspace_bytes(1, 64, 2 ** 21, 64, 4096) == 2 * 64 * 512 * 64 * 8 + 64 * 64 * 64 * 8
    sf = lambda u=G[0], prep=G[1], D=G[2], y=G[3], q=None, v=None, B=2, H=3, N=1024, NS=8, T=256, dt=BF16, \
        ws=G[4], wsb=1 << 30: lconv.lconv_fftconv_ssm_fwd(u, prep, D, y, q, v, B, H, N, NS, T, dt, ws, wsb, None)
    assert sf(dt=5) == UNSUP
    assert sf(T=300) == UNSUP
    assert sf(N=12) == UNSUP
    assert sf(B=-1) == SHAPE
    assert sf(u=None) == NULLP
    assert sf(prep=G[1] + 4) == MISAL
    assert sf(y=G[0]) == ALIAS
    assert sf(ws=None) == WSERR
    assert sf(B=0) == OK

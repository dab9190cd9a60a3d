"""C-ABI tests that need no GPU: the library loads, exports every declared symbol, answers
size queries, and rejects bad arguments with the documented status before any HIP call."""
import ctypes

import pytest

from fft_long_convolution_amd import lconv

F32, F16, BF16 = lconv.F32, lconv.F16, lconv.BF16
OK, NULLP, SHAPE, UNSUP, MISAL, ALIAS, WSERR, HIPERR, NOTPREP, SCRATCH = range(10)

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
    assert lconv.lconv_abi_version() == 8
    for s in range(10):
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
    assert lconv.lconv_filter_fft2d_bytes(256, 128, 128, BF16) == 256 * 256 * 256 * 4
    assert lconv.lconv_filter_fft2d_bytes(3, 64, 48, F16) == 3 * 256 * 256 * 4   # any sides <= 128
    assert lconv.lconv_filter_fft2d_bytes(1, 129, 128, BF16) == 0                # too large
    assert lconv.lconv_filter_fft2d_bytes(1, 128, 12, BF16) == 0                 # Ws not a multiple of 8
    assert lconv.lconv_filter_fft2d_bytes(1, 128, 128, F32) == 0                 # fp32: not built
    assert lconv.lconv_fftconv2d_workspace_bytes(8, 256, 128, 128, BF16) == 0    # one fused kernel


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
    assert lconv.lconv_fftconv2d_fwd(None, None, None, None, 0, 4, 128, 128, BF16, None, 0, None) == OK
    assert lconv.lconv_filter_fft2d(None, None, 0, 128, 128, BF16, None) == OK


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
    f = lambda u, kf, D, y, B, C, Hs, Ws, dt: lconv.lconv_fftconv2d_fwd(u, kf, D, y, B, C, Hs, Ws, dt,
                                                                         None, 0, None)
    assert f(A, Bq, C, Y, 2, 3, 256, 128, BF16) == UNSUP     # sides up to 128
    assert f(A, Bq, C, Y, 2, 3, 128, 20, BF16) == UNSUP      # columns in whole groups of 8
    assert f(A, Bq, C, Y, 2, 3, 128, 0, BF16) == UNSUP
    assert f(A, Bq, C, Y, 2, 3, 128, 128, F32) == UNSUP
    assert f(A, Bq, C, Y, 2, 3, 128, 128, 7) == UNSUP
    assert f(None, Bq, C, Y, 2, 3, 128, 128, BF16) == NULLP
    assert f(A + 2, Bq, C, Y, 2, 3, 128, 128, BF16) == MISAL
    assert f(A, Bq, C, A, 2, 3, 128, 128, BF16) == ALIAS
    assert f(A, Bq, C, Y, -2, 3, 128, 128, BF16) == SHAPE
    assert f(A, Bq, C, Y, 2, 3, -1, 128, BF16) == SHAPE
    g = lconv.lconv_filter_fft2d
    assert g(A, Y, 3, 128, 128, F32, None) == UNSUP
    assert g(A, Y, 3, 130, 128, BF16, None) == UNSUP
    assert g(None, Y, 3, 100, 64, BF16, None) == NULLP
    assert g(A + 4, Y, 3, 100, 64, BF16, None) == MISAL
    assert g(A, A, 3, 100, 64, BF16, None) == ALIAS


def test_no_device_gives_hip_error():
    """Valid arguments reach the HIP runtime; without a GPU that is LCONV_ERR_HIP."""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert fwd() == HIPERR
    # the set-up call and the allocation-free forward call ask for the current device first
    assert lconv.lconv_prepare(4096, BF16) == HIPERR
    assert lconv.lconv_fftconv_fwd_noalloc(A, Bq, C, Y, None, None, 2, 3, 64, BF16, None) == HIPERR


def test_noalloc_scratch_size():
    assert lconv.NOALLOC_SCRATCH_BYTES == 64 << 20
    # every supported length that is a multiple of 8 fits the scratch buffer with one sequence
    # per chunk: the largest transform (M = 2^23) in fp32 is exactly 64 MiB
    assert lconv.lconv_fftconv_workspace_bytes(1, 1, 2 ** 22, F32) == 64 << 20


# more fake addresses for the gradient call (1 MiB apart, far larger than the test shapes)
G = [0x10000000 + 0x100000 * i for i in range(12)]


def bwd(dy=G[0], u=G[1], kf=G[2], D=G[3], q=None, v=None, du=G[4], dq=None, dv=None, dk=None,
        dD=None, B=2, H=3, N=64, dt=BF16, ws=None, wsb=0):
    return lconv.lconv_fftconv_bwd(dy, u, kf, D, q, v, du, dq, dv, dk, dD, B, H, N, dt, ws, wsb, None)


def test_bwd_validation_errors():
    assert bwd(dt=5) == UNSUP
    assert bwd(B=-1) == SHAPE
    assert bwd(H=2 ** 40, N=2 ** 30) == SHAPE                           # overflow
    assert bwd(N=12) == UNSUP
    assert bwd(N=2 ** 22 + 8) == UNSUP
    # beyond one workgroup: the multi-pass gradient needs its workspace (fake addresses far apart)
    far = [1 << 40 + i for i in range(8)]
    big = dict(dy=far[0], u=far[1], kf=far[2], D=far[3], du=far[4], N=8192)
    need = lconv.lconv_fftconv_bwd_workspace_bytes(2, 3, 8192, BF16)
    assert need > 0
    assert bwd(**big) == WSERR
    assert bwd(**big, ws=far[5], wsb=need - 1) == WSERR
    assert bwd(**big, ws=far[5] + 8, wsb=need) == MISAL
    assert bwd(**big, ws=far[1], wsb=need) == ALIAS                        # workspace over u
    assert bwd(**big, ws=far[4] - 256, wsb=need) == ALIAS                  # workspace over du
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


def fsave(u=G[0], kf=G[1], D=G[2], y=G[3], c=G[4], q=None, v=None, B=2, H=3, N=64, dt=BF16, ws=None,
          wsb=0):
    return lconv.lconv_fftconv_fwd_save(u, kf, D, y, c, q, v, B, H, N, dt, ws, wsb, None)


def bsaved(dy=G[0], u=G[1], kf=G[2], D=G[3], q=None, v=None, c=None, du=G[4], dq=None, dv=None,
           dk=None, dD=None, B=2, H=3, N=64, dt=BF16):
    return lconv.lconv_fftconv_bwd_saved(dy, u, kf, D, q, v, c, du, dq, dv, dk, dD, B, H, N, dt, None, 0,
                                         None)


def test_forward_save_validation_errors():
    assert fsave(dt=5) == UNSUP
    assert fsave(B=-1) == SHAPE
    assert fsave(N=12) == UNSUP                                            # N % 8
    far = [1 << 40 + i for i in range(6)]
    assert fsave(u=far[0], kf=far[1], D=far[2], y=far[3], c=far[4], N=8192) == WSERR   # multi-pass: workspace
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
    assert bsaved(N=8192) == WSERR                                         # multi-pass: workspace
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


def pbwd(dy=G[0], u=G[1], kf=G[2], D=G[3], q=None, v=None, du=G[4], dq=None, dv=None, dk=None,
         dD=None, B=2, H=3, N=64, L=32, dt=BF16, ws="auto", wsb=None):
    if ws == "auto":
        wsb = lconv.lconv_fftconv_partial_bwd_workspace_bytes(B, H, N, dt) if wsb is None else wsb
        ws = G[9] if wsb else None
    return lconv.lconv_fftconv_partial_bwd(dy, u, kf, D, q, v, du, dq, dv, dk, dD, B, H, N, L, dt, ws,
                                           wsb or 0, None)


def test_partial_bwd_sizes_and_validation():
    # single pass: rev(ds) and its convolution (dtype), then the [H][N] fp32 filter gradient
    assert lconv.lconv_fftconv_partial_bwd_workspace_bytes(2, 3, 64, BF16) == 2 * 768 + 768
    assert lconv.lconv_fftconv_partial_bwd_workspace_bytes(2, 3, 64, 5) == 0
    assert lconv.lconv_fftconv_partial_bwd_workspace_bytes(0, 3, 64, BF16) == 0
    assert lconv.lconv_fftconv_partial_bwd_workspace_bytes(2, 3, 12, BF16) == 0
    assert lconv.lconv_fftconv_partial_bwd_workspace_bytes(1, 1, 2 ** 22 + 8, BF16) == 0
    # multi-pass N: at least the full gradient's workspace, plus the [H][N] fp32 part
    assert (lconv.lconv_fftconv_partial_bwd_workspace_bytes(2, 3, 8192, BF16)
            >= lconv.lconv_fftconv_bwd_workspace_bytes(2, 3, 8192, BF16) + 3 * 8192 * 4)
    assert pbwd(dt=5) == UNSUP
    assert pbwd(B=-1) == SHAPE
    assert pbwd(L=-8) == SHAPE
    assert pbwd(L=12) == UNSUP and pbwd(L=8192) == UNSUP and pbwd(L=0) == UNSUP
    assert pbwd(N=12) == UNSUP
    assert pbwd(N=2 ** 22 + 8) == UNSUP                                   # beyond the gradient's N
    assert pbwd(dy=None) == NULLP and pbwd(u=None) == NULLP and pbwd(kf=None) == NULLP
    assert pbwd(D=None) == NULLP and pbwd(du=None) == NULLP
    assert pbwd(q=G[5]) == NULLP                                          # q without dq
    assert pbwd(v=G[6]) == NULLP                                          # v without dv
    assert pbwd(ws=None, wsb=0) == WSERR
    assert pbwd(wsb=lconv.lconv_fftconv_partial_bwd_workspace_bytes(2, 3, 64, BF16) - 1) == WSERR
    assert pbwd(ws=G[9] + 8, wsb=4096) == MISAL
    assert pbwd(dk=G[7] + 4) == MISAL
    assert pbwd(du=G[0]) == ALIAS                                         # du == dy
    assert pbwd(dk=G[3]) == ALIAS                                         # dk over D
    assert pbwd(ws=G[1], wsb=4096) == ALIAS                               # workspace over u
    assert pbwd(dk=G[7], dD=G[7] + 16) == ALIAS                           # dD inside dk [H][L]
    import torch
    if not torch.cuda.is_available():                                     # valid: fails at the first HIP call
        assert pbwd(dk=G[7], dD=G[7] + 3 * 32 * 4) == HIPERR              # dD just past dk [H][L]


def test_partial_bwd_empty():
    assert pbwd(H=0) == OK
    assert pbwd(B=0, ws=None, wsb=0) == OK                                # nothing to zero
    assert pbwd(N=0, ws=None, wsb=0) == OK
    assert pbwd(B=0, dy=None, u=None, du=None, ws=None, wsb=0) == OK
    import torch
    if not torch.cuda.is_available():                                     # zero fill: a HIP call
        assert pbwd(B=0, dk=G[7], ws=None, wsb=0) == HIPERR


def bwd2d(dy=G[0], u=G[1], kf=G[2], D=G[3], du=G[4], dk=None, dD=None, B=2, C=3, Hs=16, Ws=16, dt=BF16,
          ws="auto", wsb=None):
    if ws == "auto":
        wsb = lconv.lconv_fftconv2d_bwd_workspace_bytes(B, C, Hs, Ws, dt) if wsb is None else wsb
        ws = 1 << 44 if wsb else None        # far from every other fake address
    return lconv.lconv_fftconv2d_bwd(dy, u, kf, D, du, dk, dD, B, C, Hs, Ws, dt, ws, wsb or 0, None)


def test_2d_bwd_sizes_and_validation():
    spec = 256 * 256 * 4        # one 2D spectrum (16-bit pairs)
    act = 2 * 3 * 16 * 16 * 2
    assert lconv.lconv_fftconv2d_bwd_workspace_bytes(2, 3, 16, 16, BF16) == 3 * spec + 6 * spec + act + 256
    assert lconv.lconv_fftconv2d_bwd_workspace_bytes(2, 3, 16, 16, F32) == 0
    assert lconv.lconv_fftconv2d_bwd_workspace_bytes(2, 3, 16, 12, BF16) == 0     # Ws % 8
    assert lconv.lconv_fftconv2d_bwd_workspace_bytes(2, 3, 129, 16, BF16) == 0
    assert lconv.lconv_fftconv2d_bwd_workspace_bytes(0, 3, 16, 16, BF16) == 0
    assert bwd2d(dt=F32) == UNSUP
    assert bwd2d(B=-1) == SHAPE
    assert bwd2d(Ws=12) == UNSUP and bwd2d(Hs=200) == UNSUP
    assert bwd2d(dy=None) == NULLP and bwd2d(u=None) == NULLP and bwd2d(kf=None) == NULLP
    assert bwd2d(D=None) == NULLP and bwd2d(du=None) == NULLP
    assert bwd2d(ws=None, wsb=0) == WSERR
    assert bwd2d(wsb=lconv.lconv_fftconv2d_bwd_workspace_bytes(2, 3, 16, 16, BF16) - 1) == WSERR
    assert bwd2d(dk=G[7] + 4) == MISAL
    assert bwd2d(du=G[0]) == ALIAS                                       # du == dy
    assert bwd2d(dk=G[2] + 64) == ALIAS                                  # dk over k_f
    assert bwd2d(dk=G[7], dD=G[7] + 256) == ALIAS                        # dD inside dk [C][Hs][Ws]
    assert bwd2d(ws=G[1], wsb=1 << 24) == ALIAS                          # workspace over u
    assert bwd2d(C=0) == OK
    assert bwd2d(B=0, ws=None, wsb=0) == OK                              # nothing to zero
    import torch
    if not torch.cuda.is_available():
        assert bwd2d(B=0, dk=G[7], ws=None, wsb=0) == HIPERR             # zero fill: a HIP call
        assert bwd2d(dk=G[7], dD=G[8]) == HIPERR                         # valid: first HIP call fails


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


def bfly(u=G[0], kf=G[1], D=G[2], y=G[3], q=None, v=None, tab=G[4], B=2, H=3, N=1000, dt=BF16):
    return lconv.lconv_butterfly_fwd(u, kf, D, y, q, v, tab, B, H, N, dt, None)


def test_butterfly_sizes_and_validation():
    # R = M / 256: 2 R^2 + 4 * 256 R complex block values
    assert lconv.lconv_butterfly_blocks_count(64) == 2 * 4 + 1024 * 2
    assert lconv.lconv_butterfly_blocks_count(4096) == 2 * 32 * 32 + 1024 * 32
    assert lconv.lconv_butterfly_blocks_count(8192) == 0          # beyond one transform
    assert lconv.lconv_butterfly_blocks_count(12) == 0            # not a multiple of 8
    # fp32 images (filter) + compute-type images (convolution); fp32: one set
    b32, b16 = lconv.lconv_butterfly_tables_bytes(4096, F32), lconv.lconv_butterfly_tables_bytes(4096, BF16)
    assert b32 > 0 and b16 > b32
    assert lconv.lconv_butterfly_tables_bytes(4096, 7) == 0
    assert lconv.lconv_butterfly_tables(G[0], G[1], 8192, BF16, None) == UNSUP
    assert lconv.lconv_butterfly_tables(None, G[1], 64, BF16, None) == NULLP
    assert lconv.lconv_butterfly_tables(G[0], G[0], 64, BF16, None) == ALIAS
    assert lconv.lconv_butterfly_filter(G[0], G[1], G[2], 3, 4104, BF16, None) == UNSUP
    assert lconv.lconv_butterfly_filter(G[0], G[1], None, 3, 64, BF16, None) == NULLP
    assert lconv.lconv_butterfly_filter(G[0], G[1], G[2], 0, 64, BF16, None) == OK
    assert bfly(dt=5) == UNSUP
    assert bfly(B=-1) == SHAPE
    assert bfly(N=8192) == UNSUP
    assert bfly(tab=None) == NULLP
    assert bfly(D=G[2] + 2) == MISAL
    assert bfly(y=G[0]) == ALIAS
    assert bfly(y=G[4]) == ALIAS                                   # output over the tables
    assert bfly(B=0) == OK


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


def _header_decls():
    """{name: (return type, [parameter types])} of every function include/lconv.h declares."""
    import re
    src = open(lconv.HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    out = {}
    for m in re.finditer(r"([A-Za-z_][A-Za-z0-9_ \*]*?)\b(lconv_[a-z0-9_]+)\s*\(([^;{]*?)\)\s*;", src):
        ret, name, params = " ".join(m.group(1).split()), m.group(2), m.group(3)
        types = []
        for p in params.split(","):
            p = " ".join(p.replace("*", " * ").split())
            if not p or p == "void":
                continue
            toks = p.split(" ")
            types.append(" ".join(toks[:-1]).replace(" *", "*"))   # drop the parameter name
        out[name] = (ret, types)
    return out


# The boundary's entry points with their parameter types (the filter transform also takes a
# workspace: the multi-pass filter spectrum and the staging of ragged rows need one).
BOUNDARY = {
    "lconv_filter_fft_bytes": ("size_t", ["int64_t", "int64_t", "lconv_dtype_t"]),
    "lconv_filter_fft2d_bytes": ("size_t", ["int64_t", "int64_t", "int64_t", "lconv_dtype_t"]),
    "lconv_fftconv_workspace_bytes": ("size_t", ["int64_t", "int64_t", "int64_t", "lconv_dtype_t"]),
    "lconv_fftconv2d_workspace_bytes": ("size_t", ["int64_t", "int64_t", "int64_t", "int64_t",
                                                   "lconv_dtype_t"]),
    "lconv_filter_fft": ("lconv_status_t", ["const void*", "void*", "int64_t", "int64_t", "lconv_dtype_t",
                                            "void*", "size_t", "hipStream_t"]),
    "lconv_filter_fft2d": ("lconv_status_t", ["const void*", "void*", "int64_t", "int64_t", "int64_t",
                                              "lconv_dtype_t", "hipStream_t"]),
    "lconv_fftconv_fwd": ("lconv_status_t", ["const void*", "const void*", "const void*", "void*",
                                             "const void*", "const void*", "int64_t", "int64_t", "int64_t",
                                             "lconv_dtype_t", "void*", "size_t", "hipStream_t"]),
    "lconv_fftconv2d_fwd": ("lconv_status_t", ["const void*", "const void*", "const void*", "void*",
                                               "int64_t", "int64_t", "int64_t", "int64_t", "lconv_dtype_t",
                                               "void*", "size_t", "hipStream_t"]),
    "lconv_status_string": ("const char*", ["lconv_status_t"]),
    "lconv_butterfly_tables": ("lconv_status_t", ["const void*", "void*", "int64_t", "lconv_dtype_t",
                                                  "hipStream_t"]),
    "lconv_butterfly_filter": ("lconv_status_t", ["const void*", "void*", "const void*", "int64_t", "int64_t",
                                                  "lconv_dtype_t", "hipStream_t"]),
    "lconv_butterfly_fwd": ("lconv_status_t", ["const void*", "const void*", "const void*", "void*",
                                               "const void*", "const void*", "const void*", "int64_t",
                                               "int64_t", "int64_t", "lconv_dtype_t", "hipStream_t"]),
}


def test_boundary_signatures():
    decls = _header_decls()
    for name, (ret, types) in BOUNDARY.items():
        assert name in decls, name
        assert decls[name] == (ret, types), (name, decls[name])


def test_binding_arity_matches_header(lib):
    """The ctypes binding passes exactly the parameters each declaration has."""
    decls = _header_decls()
    assert set(decls) == set(lconv.header_functions())
    for name, (_, types) in decls.items():
        assert len(getattr(lib, name).argtypes) == len(types), name

"""Python binding of liblconv.so (the gfx950 causal long-convolution library).

Argument marshalling only: every step of the computation runs in the HIP kernels behind the
C ABI declared in include/lconv.h.  torch provides device memory and the current stream.
There is no CPU fallback: if the library is missing, importing the entry points fails loudly.

Raw entry points keep the C names (``lconv_filter_fft``, ``lconv_fftconv_fwd``, ...), taking
integer device pointers.  ``filter_fft``, ``fftconv``, ``fftconv_partial``, ``fftconv_sparse``,
``fftconv_bwd``, ``fftconv_save``, ``filter_fft2d`` and ``fftconv2d`` are convenience wrappers over torch
tensors.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblconv.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "lconv.h")

F32, F16, BF16 = 0, 1, 2
STATUS = {0: "LCONV_SUCCESS", 1: "LCONV_ERR_NULL_POINTER", 2: "LCONV_ERR_INVALID_SHAPE",
          3: "LCONV_ERR_UNSUPPORTED", 4: "LCONV_ERR_MISALIGNED", 5: "LCONV_ERR_ALIASING",
          6: "LCONV_ERR_WORKSPACE", 7: "LCONV_ERR_HIP"}


class LconvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


_lib = None


def load(path: str = LIB_PATH):
    """Load liblconv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the HIP library first "
                           "(python -m fft_long_convolution_amd.build)")
    lib = ctypes.CDLL(path)
    vp, i64, sz, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    sig = {
        "lconv_filter_fft_bytes": (sz, [i64, i64, i]),
        "lconv_filter_fft_workspace_bytes": (sz, [i64, i64, i]),
        "lconv_fftconv_workspace_bytes": (sz, [i64, i64, i64, i]),
        "lconv_filter_fft2d_bytes": (sz, [i64, i64, i]),
        "lconv_filter_fft": (i, [vp, vp, i64, i64, i, vp, sz, vp]),
        "lconv_fftconv_fwd": (i, [vp, vp, vp, vp, vp, vp, i64, i64, i64, i, vp, sz, vp]),
        "lconv_fftconv_bwd": (i, [vp] * 11 + [i64, i64, i64, i, vp]),
        "lconv_fftconv_fwd_save": (i, [vp] * 7 + [i64, i64, i64, i, vp]),
        "lconv_fftconv_bwd_saved": (i, [vp] * 12 + [i64, i64, i64, i, vp]),
        "lconv_fftconv_partial_fwd": (i, [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i, vp]),
        "lconv_fftconv_sparse_fwd": (i, [vp, vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_uint32, i, vp]),
        "lconv_freq_blocks": (i, [i64]),
        "lconv_filter_fft2d": (i, [vp, vp, i64, i64, i, vp]),
        "lconv_ssm_prep_bytes": (sz, [i64, i64, i64, i]),
        "lconv_ssm_prepare": (i, [vp, vp, vp, i64, i64, i64, i, vp]),
        "lconv_fftconv_ssm_workspace_bytes": (sz, [i64, i64, i64, i64, i64]),
        "lconv_fftconv_ssm_fwd": (i, [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i, vp, sz, vp]),
        "lconv_filter_fft3d_bytes": (sz, [i64, i64, i]),
        "lconv_filter_fft3d_workspace_bytes": (sz, [i64, i64, i]),
        "lconv_fftconv3d_workspace_bytes": (sz, [i64, i64, i64, i]),
        "lconv_filter_fft3d": (i, [vp, vp, i64, i64, i, vp, sz, vp]),
        "lconv_fftconv3d_fwd": (i, [vp, vp, vp, vp, i64, i64, i64, i, vp, sz, vp]),
        "lconv_fftconv2d_fwd": (i, [vp, vp, vp, vp, i64, i64, i64, i, vp]),
        "lconv_status_string": (ctypes.c_char_p, [i]),
        "lconv_abi_version": (i, []),
        "lconv_release": (i, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def header_functions(path: str = HEADER):
    """Names of the functions declared in include/lconv.h."""
    src = open(path).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lconv_[a-z0-9_]+)\s*\(", src)))


# ---- raw C entry points (same names as the ABI) -------------------------------------------

def lconv_filter_fft_bytes(H, N, dtype):
    return load().lconv_filter_fft_bytes(H, N, dtype)


def lconv_filter_fft_workspace_bytes(H, N, dtype):
    return load().lconv_filter_fft_workspace_bytes(H, N, dtype)


def lconv_fftconv_workspace_bytes(B, H, N, dtype):
    return load().lconv_fftconv_workspace_bytes(B, H, N, dtype)


def lconv_filter_fft2d_bytes(C, S, dtype):
    return load().lconv_filter_fft2d_bytes(C, S, dtype)


def lconv_filter_fft(k, k_f, H, N, dtype, workspace, workspace_bytes, stream):
    return load().lconv_filter_fft(k, k_f, H, N, dtype, workspace, workspace_bytes, stream)


def lconv_fftconv_fwd(u, k_f, D, y, q, v, B, H, N, dtype, workspace, workspace_bytes, stream):
    return load().lconv_fftconv_fwd(u, k_f, D, y, q, v, B, H, N, dtype, workspace,
                                    workspace_bytes, stream)


def lconv_fftconv_bwd(dy, u, k_f, D, q, v, du, dq, dv, dk, dD, B, H, N, dtype, stream):
    return load().lconv_fftconv_bwd(dy, u, k_f, D, q, v, du, dq, dv, dk, dD, B, H, N, dtype, stream)


def lconv_fftconv_fwd_save(u, k_f, D, y, c, q, v, B, H, N, dtype, stream):
    return load().lconv_fftconv_fwd_save(u, k_f, D, y, c, q, v, B, H, N, dtype, stream)


def lconv_fftconv_bwd_saved(dy, u, k_f, D, q, v, c, du, dq, dv, dk, dD, B, H, N, dtype, stream):
    return load().lconv_fftconv_bwd_saved(dy, u, k_f, D, q, v, c, du, dq, dv, dk, dD, B, H, N, dtype, stream)


def lconv_fftconv_partial_fwd(u, k_f, D, y, q, v, B, H, N, L, dtype, stream):
    return load().lconv_fftconv_partial_fwd(u, k_f, D, y, q, v, B, H, N, L, dtype, stream)


def lconv_fftconv_sparse_fwd(u, k_f, D, y, q, v, B, H, N, keep, dtype, stream):
    return load().lconv_fftconv_sparse_fwd(u, k_f, D, y, q, v, B, H, N, keep, dtype, stream)


def lconv_freq_blocks(N):
    return load().lconv_freq_blocks(N)


def lconv_filter_fft2d(k, k_f, C, S, dtype, stream):
    return load().lconv_filter_fft2d(k, k_f, C, S, dtype, stream)


def lconv_fftconv2d_fwd(u, k_f, D, y, B, C, S, dtype, stream):
    return load().lconv_fftconv2d_fwd(u, k_f, D, y, B, C, S, dtype, stream)


def lconv_ssm_prep_bytes(H, NS, T, dtype):
    return load().lconv_ssm_prep_bytes(H, NS, T, dtype)


def lconv_ssm_prepare(lam, W, prep, H, NS, T, dtype, stream):
    return load().lconv_ssm_prepare(lam, W, prep, H, NS, T, dtype, stream)


def lconv_fftconv_ssm_workspace_bytes(B, H, N, NS, T):
    return load().lconv_fftconv_ssm_workspace_bytes(B, H, N, NS, T)


def lconv_fftconv_ssm_fwd(u, prep, D, y, q, v, B, H, N, NS, T, dtype, workspace, workspace_bytes, stream):
    return load().lconv_fftconv_ssm_fwd(u, prep, D, y, q, v, B, H, N, NS, T, dtype, workspace,
                                        workspace_bytes, stream)


def lconv_filter_fft3d_bytes(C, S, dtype):
    return load().lconv_filter_fft3d_bytes(C, S, dtype)


def lconv_filter_fft3d_workspace_bytes(C, S, dtype):
    return load().lconv_filter_fft3d_workspace_bytes(C, S, dtype)


def lconv_fftconv3d_workspace_bytes(B, C, S, dtype):
    return load().lconv_fftconv3d_workspace_bytes(B, C, S, dtype)


def lconv_filter_fft3d(k, k_f, C, S, dtype, workspace, workspace_bytes, stream):
    return load().lconv_filter_fft3d(k, k_f, C, S, dtype, workspace, workspace_bytes, stream)


def lconv_fftconv3d_fwd(u, k_f, D, y, B, C, S, dtype, workspace, workspace_bytes, stream):
    return load().lconv_fftconv3d_fwd(u, k_f, D, y, B, C, S, dtype, workspace, workspace_bytes, stream)


def lconv_abi_version():
    return load().lconv_abi_version()


def lconv_release():
    return load().lconv_release()


def lconv_status_string(status):
    return load().lconv_status_string(status)


def status_string(status: int) -> str:
    return lconv_status_string(status).decode()


# ---- torch wrappers ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    return {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}[t]


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(status, where):
    if status != 0:
        raise LconvError(status, where)


def filter_fft(k, stream=None):
    """Opaque filter spectrum (uint8 device tensor) for k [H, N]."""
    torch = _torch()
    H, N = k.shape
    dt = dtype_code(k.dtype)
    nbytes = lconv_filter_fft_bytes(H, N, dt)
    if nbytes == 0 and H * N > 0:
        raise LconvError(3, "lconv_filter_fft_bytes")
    k_f = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=k.device)
    wsb = lconv_filter_fft_workspace_bytes(H, N, dt)
    ws = torch.empty(wsb, dtype=torch.uint8, device=k.device) if wsb else None
    _check(lconv_filter_fft(_ptr(k), k_f.data_ptr(), H, N, dt, _ptr(ws), wsb, _stream(stream)),
           "lconv_filter_fft")
    return k_f


def fftconv(u, k_f, D, q=None, v=None, out=None, stream=None):
    """y = v * ((k * (q*u))[:N] + D * (q*u)) for u [B, H, N]."""
    torch = _torch()
    B, H, N = u.shape
    dt = dtype_code(u.dtype)
    y = torch.empty_like(u) if out is None else out
    wsb = lconv_fftconv_workspace_bytes(B, H, N, dt)
    ws = torch.empty(wsb, dtype=torch.uint8, device=u.device) if wsb else None
    _check(lconv_fftconv_fwd(_ptr(u), _ptr(k_f), _ptr(D), _ptr(y), _ptr(q), _ptr(v), B, H, N, dt,
                             _ptr(ws), wsb, _stream(stream)), "lconv_fftconv_fwd")
    return y


def fftconv_save(u, k_f, D, q=None, v=None, stream=None):
    """(y, c): y = v * c with the pre-gate output c = (k * (q*u))[:N] + D * (q*u), for the
    gradient call (N <= 4096)."""
    torch = _torch()
    B, H, N = u.shape
    dt = dtype_code(u.dtype)
    y = torch.empty_like(u)
    c = torch.empty_like(u)
    _check(lconv_fftconv_fwd_save(_ptr(u), _ptr(k_f), _ptr(D), _ptr(y), _ptr(c), _ptr(q), _ptr(v),
                                  B, H, N, dt, _stream(stream)), "lconv_fftconv_fwd_save")
    return y, c


def fftconv_bwd(dy, u, k_f, D, q=None, v=None, need_dk=True, c=None, stream=None):
    """Gradients of y = v * ((k * (q*u))[:N] + D * (q*u)) given dy [B, H, N].

    With c (the pre-gate output from fftconv_save), dv = dy * c without a transform.
    Returns (du, dq, dv, dk, dD): du, dq, dv in u's dtype (dq is None without q, dv is None
    without v); dk [H, N] and dD [H] in float32 (None when need_dk is False)."""
    torch = _torch()
    B, H, N = u.shape
    dt = dtype_code(u.dtype)
    du = torch.empty_like(u)
    dq = torch.empty_like(u) if q is not None else None
    dv = torch.empty_like(u) if v is not None else None
    dk = torch.empty((H, N), dtype=torch.float32, device=u.device) if need_dk else None
    dD = torch.empty((H,), dtype=torch.float32, device=u.device) if need_dk else None
    if c is None:
        _check(lconv_fftconv_bwd(_ptr(dy), _ptr(u), _ptr(k_f), _ptr(D), _ptr(q), _ptr(v), _ptr(du),
                                 _ptr(dq), _ptr(dv), _ptr(dk), _ptr(dD), B, H, N, dt, _stream(stream)),
               "lconv_fftconv_bwd")
    else:
        _check(lconv_fftconv_bwd_saved(_ptr(dy), _ptr(u), _ptr(k_f), _ptr(D), _ptr(q), _ptr(v), _ptr(c),
                                       _ptr(du), _ptr(dq), _ptr(dv), _ptr(dk), _ptr(dD), B, H, N, dt,
                                       _stream(stream)), "lconv_fftconv_bwd_saved")
    return du, dq, dv, dk, dD


def fftconv_partial(u, k_f, D, L, q=None, v=None, out=None, stream=None):
    """y = v * ((k * (q*u))[:N] + D * (q*u)) for a filter of L taps (k_f = filter_fft(k [H, L]))
    and u [B, H, N] of any length N."""
    torch = _torch()
    B, H, N = u.shape
    y = torch.empty_like(u) if out is None else out
    _check(lconv_fftconv_partial_fwd(_ptr(u), _ptr(k_f), _ptr(D), _ptr(y), _ptr(q), _ptr(v), B, H, N,
                                     L, dtype_code(u.dtype), _stream(stream)),
           "lconv_fftconv_partial_fwd")
    return y


def fftconv_sparse(u, k_f, D, keep, q=None, v=None, out=None, stream=None):
    """Frequency-sparse convolution: as fftconv, with the filter spectrum kept only on the
    frequency blocks r (f mod R = r, R = lconv_freq_blocks(N)) in `keep` (an iterable of block
    indices closed under r -> R - r, or a bit mask)."""
    torch = _torch()
    B, H, N = u.shape
    mask = keep if isinstance(keep, int) else sum(1 << int(r) for r in set(keep))
    y = torch.empty_like(u) if out is None else out
    _check(lconv_fftconv_sparse_fwd(_ptr(u), _ptr(k_f), _ptr(D), _ptr(y), _ptr(q), _ptr(v), B, H, N,
                                    mask, dtype_code(u.dtype), _stream(stream)),
           "lconv_fftconv_sparse_fwd")
    return y


def filter_fft2d(k, stream=None):
    torch = _torch()
    C, S, _ = k.shape
    dt = dtype_code(k.dtype)
    nbytes = lconv_filter_fft2d_bytes(C, S, dt)
    k_f = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=k.device)
    _check(lconv_filter_fft2d(_ptr(k), k_f.data_ptr(), C, S, dt, _stream(stream)), "lconv_filter_fft2d")
    return k_f


def ssm_prepare(lam, W, T, dtype, stream=None):
    """Tables for the state-space filter k[h, t] = Re sum_n W lam^t: lam, W complex64 device
    tensors [H, NS]; T the chunk length.  Returns the opaque prep buffer."""
    torch = _torch()
    H, NS = lam.shape
    dt = dtype_code(dtype)
    nbytes = lconv_ssm_prep_bytes(H, NS, T, dt)
    if nbytes == 0:
        raise LconvError(3, "lconv_ssm_prep_bytes")
    prep = torch.empty(nbytes, dtype=torch.uint8, device=lam.device)
    lam_f = torch.view_as_real(lam.contiguous()).contiguous()
    W_f = torch.view_as_real(W.contiguous()).contiguous()
    _check(lconv_ssm_prepare(lam_f.data_ptr(), W_f.data_ptr(), prep.data_ptr(), H, NS, T, dt, _stream(stream)),
           "lconv_ssm_prepare")
    return prep


def fftconv_ssm(u, prep, D, NS, T, q=None, v=None, out=None, stream=None):
    """Causal convolution with a state-space filter, chunked with state passing."""
    torch = _torch()
    B, H, N = u.shape
    y = torch.empty_like(u) if out is None else out
    wsb = lconv_fftconv_ssm_workspace_bytes(B, H, N, NS, T)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=u.device)
    _check(lconv_fftconv_ssm_fwd(_ptr(u), _ptr(prep), _ptr(D), _ptr(y), _ptr(q), _ptr(v), B, H, N, NS, T,
                                 dtype_code(u.dtype), ws.data_ptr(), wsb, _stream(stream)),
           "lconv_fftconv_ssm_fwd")
    return y


def filter_fft3d(k, stream=None):
    """Opaque 3D filter spectrum for k [C, S, S, S]."""
    torch = _torch()
    C, S = k.shape[0], k.shape[1]
    dt = dtype_code(k.dtype)
    k_f = torch.empty(max(lconv_filter_fft3d_bytes(C, S, dt), 1), dtype=torch.uint8, device=k.device)
    wsb = lconv_filter_fft3d_workspace_bytes(C, S, dt)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=k.device)
    _check(lconv_filter_fft3d(_ptr(k), k_f.data_ptr(), C, S, dt, ws.data_ptr(), wsb, _stream(stream)),
           "lconv_filter_fft3d")
    return k_f


def fftconv3d(u, k_f, D, out=None, stream=None):
    """3D centred linear convolution plus skip for u [B, C, S, S, S]."""
    torch = _torch()
    B, C, S = u.shape[:3]
    dt = dtype_code(u.dtype)
    y = torch.empty_like(u) if out is None else out
    wsb = lconv_fftconv3d_workspace_bytes(B, C, S, dt)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=u.device)
    _check(lconv_fftconv3d_fwd(_ptr(u), _ptr(k_f), _ptr(D), _ptr(y), B, C, S, dt, ws.data_ptr(), wsb,
                               _stream(stream)), "lconv_fftconv3d_fwd")
    return y


def fftconv2d(u, k_f, D, out=None, stream=None):
    torch = _torch()
    B, C, S, _ = u.shape
    dt = dtype_code(u.dtype)
    y = torch.empty_like(u) if out is None else out
    _check(lconv_fftconv2d_fwd(_ptr(u), _ptr(k_f), _ptr(D), _ptr(y), B, C, S, dt, _stream(stream)),
           "lconv_fftconv2d_fwd")
    return y

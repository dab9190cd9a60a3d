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
          6: "LCONV_ERR_WORKSPACE", 7: "LCONV_ERR_HIP", 8: "LCONV_ERR_NOT_PREPARED",
          9: "LCONV_ERR_SCRATCH_LIMIT"}
NOALLOC_SCRATCH_BYTES = 64 << 20   # LCONV_NOALLOC_SCRATCH_BYTES


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
        "lconv_filter_fft2d_bytes": (sz, [i64, i64, i64, i]),
        "lconv_fftconv2d_workspace_bytes": (sz, [i64, i64, i64, i64, i]),
        "lconv_filter_fft": (i, [vp, vp, i64, i64, i, vp, sz, vp]),
        "lconv_fftconv_fwd": (i, [vp, vp, vp, vp, vp, vp, i64, i64, i64, i, vp, sz, vp]),
        "lconv_fftconv_bwd_workspace_bytes": (sz, [i64, i64, i64, i]),
        "lconv_fftconv_bwd": (i, [vp] * 11 + [i64, i64, i64, i, vp, sz, vp]),
        "lconv_fftconv_fwd_save": (i, [vp] * 7 + [i64, i64, i64, i, vp, sz, vp]),
        "lconv_fftconv_bwd_saved": (i, [vp] * 12 + [i64, i64, i64, i, vp, sz, vp]),
        "lconv_fftconv_partial_fwd": (i, [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i, vp]),
        "lconv_fftconv_partial_bwd_workspace_bytes": (sz, [i64, i64, i64, i]),
        "lconv_fftconv_partial_bwd": (i, [vp] * 11 + [i64, i64, i64, i64, i, vp, sz, vp]),
        "lconv_fftconv_sparse_fwd": (i, [vp, vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_uint32, i, vp]),
        "lconv_freq_blocks": (i, [i64]),
        "lconv_butterfly_blocks_count": (i64, [i64]),
        "lconv_butterfly_tables_bytes": (sz, [i64, i]),
        "lconv_butterfly_tables": (i, [vp, vp, i64, i, vp]),
        "lconv_butterfly_filter": (i, [vp, vp, vp, i64, i64, i, vp]),
        "lconv_butterfly_fwd": (i, [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i, vp]),
        "lconv_filter_fft2d": (i, [vp, vp, i64, i64, i64, i, vp]),
        "lconv_fftconv2d_bwd_workspace_bytes": (sz, [i64, i64, i64, i64, i]),
        "lconv_fftconv2d_bwd": (i, [vp] * 7 + [i64, i64, i64, i64, i, vp, sz, vp]),
        "lconv_ssm_prep_bytes": (sz, [i64, i64, i64, i]),
        "lconv_ssm_prepare": (i, [vp, vp, vp, i64, i64, i64, i, vp]),
        "lconv_fftconv_ssm_workspace_bytes": (sz, [i64, i64, i64, i64, i64]),
        "lconv_fftconv_ssm_fwd": (i, [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i, vp, sz, vp]),
        "lconv_filter_fft3d_bytes": (sz, [i64, i64, i]),
        "lconv_filter_fft3d_workspace_bytes": (sz, [i64, i64, i]),
        "lconv_fftconv3d_workspace_bytes": (sz, [i64, i64, i64, i]),
        "lconv_filter_fft3d": (i, [vp, vp, i64, i64, i, vp, sz, vp]),
        "lconv_fftconv3d_fwd": (i, [vp, vp, vp, vp, i64, i64, i64, i, vp, sz, vp]),
        "lconv_fftconv2d_fwd": (i, [vp, vp, vp, vp, i64, i64, i64, i64, i, vp, sz, vp]),
        "lconv_prepare": (i, [i64, i]),
        "lconv_fftconv_fwd_noalloc": (i, [vp, vp, vp, vp, vp, vp, i64, i64, i64, i, vp]),
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


def lconv_filter_fft2d_bytes(C, Hs, Ws, dtype):
    return load().lconv_filter_fft2d_bytes(C, Hs, Ws, dtype)


def lconv_fftconv2d_workspace_bytes(B, C, Hs, Ws, dtype):
    return load().lconv_fftconv2d_workspace_bytes(B, C, Hs, Ws, dtype)


def lconv_filter_fft(k, k_f, H, N, dtype, workspace, workspace_bytes, stream):
    return load().lconv_filter_fft(k, k_f, H, N, dtype, workspace, workspace_bytes, stream)


def lconv_fftconv_fwd(u, k_f, D, y, q, v, B, H, N, dtype, workspace, workspace_bytes, stream):
    return load().lconv_fftconv_fwd(u, k_f, D, y, q, v, B, H, N, dtype, workspace,
                                    workspace_bytes, stream)


def lconv_prepare(N, dtype):
    return load().lconv_prepare(N, dtype)


def lconv_fftconv_fwd_noalloc(u, k_f, D, y, q, v, B, H, N, dtype, stream):
    return load().lconv_fftconv_fwd_noalloc(u, k_f, D, y, q, v, B, H, N, dtype, stream)


def lconv_fftconv_bwd_workspace_bytes(B, H, N, dtype):
    return load().lconv_fftconv_bwd_workspace_bytes(B, H, N, dtype)


def lconv_fftconv_bwd(dy, u, k_f, D, q, v, du, dq, dv, dk, dD, B, H, N, dtype, workspace, workspace_bytes,
                      stream):
    return load().lconv_fftconv_bwd(dy, u, k_f, D, q, v, du, dq, dv, dk, dD, B, H, N, dtype, workspace,
                                    workspace_bytes, stream)


def lconv_fftconv_fwd_save(u, k_f, D, y, c, q, v, B, H, N, dtype, workspace, workspace_bytes, stream):
    return load().lconv_fftconv_fwd_save(u, k_f, D, y, c, q, v, B, H, N, dtype, workspace, workspace_bytes,
                                         stream)


def lconv_fftconv_bwd_saved(dy, u, k_f, D, q, v, c, du, dq, dv, dk, dD, B, H, N, dtype, workspace,
                            workspace_bytes, stream):
    return load().lconv_fftconv_bwd_saved(dy, u, k_f, D, q, v, c, du, dq, dv, dk, dD, B, H, N, dtype,
                                          workspace, workspace_bytes, stream)


def lconv_fftconv_partial_fwd(u, k_f, D, y, q, v, B, H, N, L, dtype, stream):
    return load().lconv_fftconv_partial_fwd(u, k_f, D, y, q, v, B, H, N, L, dtype, stream)


def lconv_fftconv_partial_bwd_workspace_bytes(B, H, N, dtype):
    return load().lconv_fftconv_partial_bwd_workspace_bytes(B, H, N, dtype)


def lconv_fftconv_partial_bwd(dy, u, k_f, D, q, v, du, dq, dv, dk, dD, B, H, N, L, dtype, workspace,
                              workspace_bytes, stream):
    return load().lconv_fftconv_partial_bwd(dy, u, k_f, D, q, v, du, dq, dv, dk, dD, B, H, N, L, dtype,
                                            workspace, workspace_bytes, stream)


def lconv_fftconv_sparse_fwd(u, k_f, D, y, q, v, B, H, N, keep, dtype, stream):
    return load().lconv_fftconv_sparse_fwd(u, k_f, D, y, q, v, B, H, N, keep, dtype, stream)


def lconv_butterfly_blocks_count(N):
    return load().lconv_butterfly_blocks_count(N)


def lconv_butterfly_tables_bytes(N, dtype):
    return load().lconv_butterfly_tables_bytes(N, dtype)


def lconv_butterfly_tables(blocks, tables, N, dtype, stream):
    return load().lconv_butterfly_tables(blocks, tables, N, dtype, stream)


def lconv_butterfly_filter(k, k_f, tables, H, N, dtype, stream):
    return load().lconv_butterfly_filter(k, k_f, tables, H, N, dtype, stream)


def lconv_butterfly_fwd(u, k_f, D, y, q, v, tables, B, H, N, dtype, stream):
    return load().lconv_butterfly_fwd(u, k_f, D, y, q, v, tables, B, H, N, dtype, stream)


def lconv_freq_blocks(N):
    return load().lconv_freq_blocks(N)


def lconv_filter_fft2d(k, k_f, C, Hs, Ws, dtype, stream):
    return load().lconv_filter_fft2d(k, k_f, C, Hs, Ws, dtype, stream)


def lconv_fftconv2d_fwd(u, k_f, D, y, B, C, Hs, Ws, dtype, workspace, workspace_bytes, stream):
    return load().lconv_fftconv2d_fwd(u, k_f, D, y, B, C, Hs, Ws, dtype, workspace, workspace_bytes, stream)


def lconv_fftconv2d_bwd_workspace_bytes(B, C, Hs, Ws, dtype):
    return load().lconv_fftconv2d_bwd_workspace_bytes(B, C, Hs, Ws, dtype)


def lconv_fftconv2d_bwd(dy, u, k_f, D, du, dk, dD, B, C, Hs, Ws, dtype, workspace, workspace_bytes, stream):
    return load().lconv_fftconv2d_bwd(dy, u, k_f, D, du, dk, dD, B, C, Hs, Ws, dtype, workspace,
                                      workspace_bytes, stream)


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


def _need(name, t, shape, dtype, optional=False):
    """Host-side checks the C ABI cannot make on a torch tensor: the dtype, the shape and a dense
    layout (the kernels read memory as contiguous rows, so a transposed or strided view would be
    read wrongly, not rejected).  The device is checked by _on_gpu once every operand passed."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (a strided or transposed view would be read as dense rows)")


def _need_buf(name, t, nbytes):
    """An opaque library buffer (filter spectrum, state-space tables): a contiguous 1-D uint8
    tensor of exactly the size the library's size query gives for this shape and dtype (a buffer
    made for another shape or dtype would be read out of bounds)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.dtype != torch.uint8 or t.dim() != 1:
        raise ValueError(f"{name} must be the 1-D uint8 tensor the library wrote")
    if t.numel() not in (nbytes, max(nbytes, 1)):
        raise ValueError(f"{name} holds {t.numel()} bytes; this shape and dtype need {nbytes} "
                         "(it was made for another shape or dtype)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(**operands):
    """Every given operand is a GPU tensor, all on the same device; returns that device."""
    dev = None
    for name, t in operands.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor, got device {t.device}")
        if dev is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other operands on {dev}")
        dev = t.device
    return dev


def _act(u, name="u", dims=3):
    """(torch dtype, shape) of the activation that fixes the call's shape."""
    torch = _torch()
    if not isinstance(u, torch.Tensor) or u.dim() != dims:
        raise ValueError(f"{name} must be a {dims}-D torch tensor")
    if u.dtype not in (torch.float32, torch.float16, torch.bfloat16):
        raise ValueError(f"{name} has dtype {u.dtype}; supported: float32, float16, bfloat16")
    _need(name, u, u.shape, u.dtype)
    return u.dtype, tuple(u.shape)


def filter_fft(k, stream=None):
    """Opaque filter spectrum (uint8 device tensor) for k [H, N]."""
    torch = _torch()
    _act(k, "k", dims=2)
    _on_gpu(k=k)
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


def _gated_inputs(u, k_f, D, q, v, out, L=None, **more):
    """Checks of the 1D calls' operands; the spectrum was made for [H, L] (L = N if None).
    `more`: further [B, H, N] operands of u's dtype (None: absent)."""
    tdt, (B, H, N) = _act(u)
    _need("D", D, (H,), tdt)
    _need("q", q, (B, H, N), tdt, optional=True)
    _need("v", v, (B, H, N), tdt, optional=True)
    _need("out", out, (B, H, N), tdt, optional=True)
    for name, t in more.items():
        _need(name, t, (B, H, N), tdt, optional=True)
    _need_buf("k_f", k_f, lconv_filter_fft_bytes(H, N if L is None else L, dtype_code(tdt)))
    _on_gpu(u=u, k_f=k_f, D=D, q=q, v=v, out=out, **more)
    return B, H, N


def fftconv(u, k_f, D, q=None, v=None, out=None, stream=None):
    """y = v * ((k * (q*u))[:N] + D * (q*u)) for u [B, H, N]."""
    torch = _torch()
    B, H, N = _gated_inputs(u, k_f, D, q, v, out)
    dt = dtype_code(u.dtype)
    y = torch.empty_like(u) if out is None else out
    wsb = lconv_fftconv_workspace_bytes(B, H, N, dt)
    ws = torch.empty(wsb, dtype=torch.uint8, device=u.device) if wsb else None
    _check(lconv_fftconv_fwd(_ptr(u), _ptr(k_f), _ptr(D), _ptr(y), _ptr(q), _ptr(v), B, H, N, dt,
                             _ptr(ws), wsb, _stream(stream)), "lconv_fftconv_fwd")
    return y


def fftconv_save(u, k_f, D, q=None, v=None, stream=None):
    """(y, c): y = v * c with the pre-gate output c = (k * (q*u))[:N] + D * (q*u), for the
    gradient call."""
    torch = _torch()
    B, H, N = _gated_inputs(u, k_f, D, q, v, None)
    dt = dtype_code(u.dtype)
    y = torch.empty_like(u)
    c = torch.empty_like(u)
    wsb = lconv_fftconv_workspace_bytes(B, H, N, dt)
    ws = torch.empty(wsb, dtype=torch.uint8, device=u.device) if wsb else None
    _check(lconv_fftconv_fwd_save(_ptr(u), _ptr(k_f), _ptr(D), _ptr(y), _ptr(c), _ptr(q), _ptr(v),
                                  B, H, N, dt, _ptr(ws), wsb, _stream(stream)), "lconv_fftconv_fwd_save")
    return y, c


def fftconv_bwd(dy, u, k_f, D, q=None, v=None, need_dk=True, c=None, stream=None):
    """Gradients of y = v * ((k * (q*u))[:N] + D * (q*u)) given dy [B, H, N].

    With c (the pre-gate output from fftconv_save), dv = dy * c without a transform.
    Returns (du, dq, dv, dk, dD): du, dq, dv in u's dtype (dq is None without q, dv is None
    without v); dk [H, N] and dD [H] in float32 (None when need_dk is False)."""
    torch = _torch()
    if dy is None:
        raise ValueError("dy is required")
    B, H, N = _gated_inputs(u, k_f, D, q, v, None, dy=dy, c=c)
    dt = dtype_code(u.dtype)
    du = torch.empty_like(u)
    dq = torch.empty_like(u) if q is not None else None
    dv = torch.empty_like(u) if v is not None else None
    dk = torch.empty((H, N), dtype=torch.float32, device=u.device) if need_dk else None
    dD = torch.empty((H,), dtype=torch.float32, device=u.device) if need_dk else None
    wsb = lconv_fftconv_bwd_workspace_bytes(B, H, N, dt)
    ws = torch.empty(wsb, dtype=torch.uint8, device=u.device) if wsb else None
    if c is None:
        _check(lconv_fftconv_bwd(_ptr(dy), _ptr(u), _ptr(k_f), _ptr(D), _ptr(q), _ptr(v), _ptr(du),
                                 _ptr(dq), _ptr(dv), _ptr(dk), _ptr(dD), B, H, N, dt, _ptr(ws), wsb,
                                 _stream(stream)), "lconv_fftconv_bwd")
    else:
        _check(lconv_fftconv_bwd_saved(_ptr(dy), _ptr(u), _ptr(k_f), _ptr(D), _ptr(q), _ptr(v), _ptr(c),
                                       _ptr(du), _ptr(dq), _ptr(dv), _ptr(dk), _ptr(dD), B, H, N, dt,
                                       _ptr(ws), wsb, _stream(stream)), "lconv_fftconv_bwd_saved")
    return du, dq, dv, dk, dD


def fftconv_partial(u, k_f, D, L, q=None, v=None, out=None, stream=None):
    """y = v * ((k * (q*u))[:N] + D * (q*u)) for a filter of L taps (k_f = filter_fft(k [H, L]))
    and u [B, H, N] of any length N."""
    torch = _torch()
    B, H, N = _gated_inputs(u, k_f, D, q, v, out, L=L)
    y = torch.empty_like(u) if out is None else out
    _check(lconv_fftconv_partial_fwd(_ptr(u), _ptr(k_f), _ptr(D), _ptr(y), _ptr(q), _ptr(v), B, H, N,
                                     L, dtype_code(u.dtype), _stream(stream)),
           "lconv_fftconv_partial_fwd")
    return y


def fftconv_partial_bwd(dy, u, k_f, D, L, q=None, v=None, need_dk=True, stream=None):
    """Gradients of fftconv_partial (a filter of L taps, k_f = filter_fft(k [H, L])) given dy
    [B, H, N].  Returns (du, dq, dv, dk, dD): du, dq, dv in u's dtype (dq None without q, dv None
    without v); dk [H, L] and dD [H] in float32 (None when need_dk is False)."""
    torch = _torch()
    if dy is None:
        raise ValueError("dy is required")
    B, H, N = _gated_inputs(u, k_f, D, q, v, None, L=L, dy=dy)
    dt = dtype_code(u.dtype)
    du = torch.empty_like(u)
    dq = torch.empty_like(u) if q is not None else None
    dv = torch.empty_like(u) if v is not None else None
    dk = torch.empty((H, L), dtype=torch.float32, device=u.device) if need_dk else None
    dD = torch.empty((H,), dtype=torch.float32, device=u.device) if need_dk else None
    wsb = lconv_fftconv_partial_bwd_workspace_bytes(B, H, N, dt)
    ws = torch.empty(wsb, dtype=torch.uint8, device=u.device) if wsb else None
    _check(lconv_fftconv_partial_bwd(_ptr(dy), _ptr(u), _ptr(k_f), _ptr(D), _ptr(q), _ptr(v), _ptr(du),
                                     _ptr(dq), _ptr(dv), _ptr(dk), _ptr(dD), B, H, N, L, dt, _ptr(ws), wsb,
                                     _stream(stream)), "lconv_fftconv_partial_bwd")
    return du, dq, dv, dk, dD


def fftconv_sparse(u, k_f, D, keep, q=None, v=None, out=None, stream=None):
    """Frequency-sparse convolution: as fftconv, with the filter spectrum kept only on the
    frequency blocks r (f mod R = r, R = lconv_freq_blocks(N)) in `keep` (an iterable of block
    indices closed under r -> R - r, or a bit mask)."""
    torch = _torch()
    B, H, N = _gated_inputs(u, k_f, D, q, v, out)
    mask = keep if isinstance(keep, int) else sum(1 << int(r) for r in set(keep))
    y = torch.empty_like(u) if out is None else out
    _check(lconv_fftconv_sparse_fwd(_ptr(u), _ptr(k_f), _ptr(D), _ptr(y), _ptr(q), _ptr(v), B, H, N,
                                    mask, dtype_code(u.dtype), _stream(stream)),
           "lconv_fftconv_sparse_fwd")
    return y


def butterfly_tables(blocks, N, dtype, stream=None):
    """Matrix-core images (uint8 device tensor) of learned-Butterfly factor blocks for length N:
    `blocks` a complex64 device tensor of lconv_butterfly_blocks_count(N) values (A1, A2, A3,
    B1, B2, B3 back to back, as include/lconv.h lays them out); dtype a torch dtype."""
    torch = _torch()
    dt = dtype_code(dtype)
    count = lconv_butterfly_blocks_count(N)
    if count == 0:
        raise LconvError(4, "lconv_butterfly_blocks_count")
    _need("blocks", blocks, (count,), torch.complex64)
    _on_gpu(blocks=blocks)
    nbytes = lconv_butterfly_tables_bytes(N, dt)
    tables = torch.empty(nbytes, dtype=torch.uint8, device=blocks.device)
    _check(lconv_butterfly_tables(blocks.data_ptr(), tables.data_ptr(), N, dt, _stream(stream)),
           "lconv_butterfly_tables")
    return tables


def butterfly_filter(k, tables, stream=None):
    """Filter spectrum of k [H, N] through the learned forward factors (same opaque layout as
    filter_fft)."""
    torch = _torch()
    _act(k, "k", dims=2)
    H, N = k.shape
    dt = dtype_code(k.dtype)
    _need_buf("tables", tables, lconv_butterfly_tables_bytes(N, dt))
    _on_gpu(k=k, tables=tables)
    nbytes = lconv_filter_fft_bytes(H, N, dt)
    if nbytes == 0 and H * N > 0:
        raise LconvError(3, "lconv_filter_fft_bytes")
    k_f = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=k.device)
    _check(lconv_butterfly_filter(_ptr(k), k_f.data_ptr(), tables.data_ptr(), H, N, dt, _stream(stream)),
           "lconv_butterfly_filter")
    return k_f


def butterfly(u, k_f, D, tables, q=None, v=None, out=None, stream=None):
    """Learned-Butterfly convolution y = v * (Re(S (K . T (q*u)))[:N] + D (q*u)) for u [B, H, N],
    k_f from butterfly_filter, tables from butterfly_tables."""
    torch = _torch()
    B, H, N = _gated_inputs(u, k_f, D, q, v, out)
    dt = dtype_code(u.dtype)
    _need_buf("tables", tables, lconv_butterfly_tables_bytes(N, dt))
    _on_gpu(tables=tables)
    y = torch.empty_like(u) if out is None else out
    _check(lconv_butterfly_fwd(_ptr(u), _ptr(k_f), _ptr(D), _ptr(y), _ptr(q), _ptr(v), tables.data_ptr(),
                               B, H, N, dt, _stream(stream)), "lconv_butterfly_fwd")
    return y


def filter_fft2d(k, stream=None):
    """Opaque 2D filter spectrum for centred kernels k [C, Hs, Ws]."""
    torch = _torch()
    _act(k, "k", dims=3)
    _on_gpu(k=k)
    C, Hs, Ws = k.shape
    dt = dtype_code(k.dtype)
    nbytes = lconv_filter_fft2d_bytes(C, Hs, Ws, dt)
    if nbytes == 0 and C > 0:
        raise LconvError(3, "lconv_filter_fft2d_bytes")
    k_f = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=k.device)
    _check(lconv_filter_fft2d(_ptr(k), k_f.data_ptr(), C, Hs, Ws, dt, _stream(stream)), "lconv_filter_fft2d")
    return k_f


def ssm_prepare(lam, W, T, dtype, stream=None):
    """Tables for the state-space filter k[h, t] = Re sum_n W lam^t: lam, W complex64 device
    tensors [H, NS]; T the chunk length.  Returns the opaque prep buffer."""
    torch = _torch()
    if not isinstance(lam, torch.Tensor) or lam.dim() != 2:
        raise ValueError("lam must be a 2-D complex64 tensor [H, NS]")
    H, NS = lam.shape
    _need("lam", lam, (H, NS), torch.complex64)
    _need("W", W, (H, NS), torch.complex64)
    _on_gpu(lam=lam, W=W)
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
    tdt, (B, H, N) = _act(u)
    _need("D", D, (H,), tdt)
    _need("q", q, (B, H, N), tdt, optional=True)
    _need("v", v, (B, H, N), tdt, optional=True)
    _need("out", out, (B, H, N), tdt, optional=True)
    _need_buf("prep", prep, lconv_ssm_prep_bytes(H, NS, T, dtype_code(tdt)))
    _on_gpu(u=u, prep=prep, D=D, q=q, v=v, out=out)
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
    _act(k, "k", dims=4)
    _on_gpu(k=k)
    C, S = k.shape[0], k.shape[1]
    if tuple(k.shape) != (C, S, S, S):
        raise ValueError(f"k has shape {tuple(k.shape)}, expected a cube [C, S, S, S]")
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
    tdt, shape = _act(u, dims=5)
    B, C, S = shape[:3]
    if shape != (B, C, S, S, S):
        raise ValueError(f"u has shape {shape}, expected [B, C, S, S, S]")
    dt = dtype_code(tdt)
    _need("D", D, (C,), tdt)
    _need("out", out, shape, tdt, optional=True)
    _need_buf("k_f", k_f, lconv_filter_fft3d_bytes(C, S, dt))
    _on_gpu(u=u, k_f=k_f, D=D, out=out)
    y = torch.empty_like(u) if out is None else out
    wsb = lconv_fftconv3d_workspace_bytes(B, C, S, dt)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=u.device)
    _check(lconv_fftconv3d_fwd(_ptr(u), _ptr(k_f), _ptr(D), _ptr(y), B, C, S, dt, ws.data_ptr(), wsb,
                               _stream(stream)), "lconv_fftconv3d_fwd")
    return y


def fftconv2d(u, k_f, D, out=None, stream=None):
    """2D centred linear convolution plus skip for u [B, C, Hs, Ws]."""
    torch = _torch()
    tdt, (B, C, Hs, Ws) = _act(u, dims=4)
    dt = dtype_code(tdt)
    _need("D", D, (C,), tdt)
    _need("out", out, (B, C, Hs, Ws), tdt, optional=True)
    _need_buf("k_f", k_f, lconv_filter_fft2d_bytes(C, Hs, Ws, dt))
    dev = _on_gpu(u=u, k_f=k_f, D=D, out=out)
    y = torch.empty_like(u) if out is None else out
    wsb = lconv_fftconv2d_workspace_bytes(B, C, Hs, Ws, dt)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
    _check(lconv_fftconv2d_fwd(_ptr(u), _ptr(k_f), _ptr(D), _ptr(y), B, C, Hs, Ws, dt, _ptr(ws), wsb,
                               _stream(stream)), "lconv_fftconv2d_fwd")
    return y


def fftconv2d_bwd(dy, u, k_f, D, need_dk=True, stream=None):
    """Gradients of fftconv2d given dy [B, C, Hs, Ws]: (du in u's dtype, dk [C, Hs, Ws] and dD [C]
    in float32; dk and dD are None when need_dk is False)."""
    torch = _torch()
    tdt, (B, C, Hs, Ws) = _act(u, dims=4)
    dt = dtype_code(tdt)
    _need("dy", dy, (B, C, Hs, Ws), tdt)
    _need("D", D, (C,), tdt)
    _need_buf("k_f", k_f, lconv_filter_fft2d_bytes(C, Hs, Ws, dt))
    dev = _on_gpu(dy=dy, u=u, k_f=k_f, D=D)
    du = torch.empty_like(u)
    dk = torch.empty((C, Hs, Ws), dtype=torch.float32, device=dev) if need_dk else None
    dD = torch.empty((C,), dtype=torch.float32, device=dev) if need_dk else None
    wsb = lconv_fftconv2d_bwd_workspace_bytes(B, C, Hs, Ws, dt)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
    _check(lconv_fftconv2d_bwd(_ptr(dy), _ptr(u), _ptr(k_f), _ptr(D), _ptr(du), _ptr(dk), _ptr(dD), B, C, Hs, Ws,
                               dt, _ptr(ws), wsb, _stream(stream)), "lconv_fftconv2d_bwd")
    return du, dk, dD

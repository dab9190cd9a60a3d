"""float64 CPU oracle: ctypes wrappers over oracle.c plus a naive-DFT 2D oracle in numpy.

TEST INFRASTRUCTURE ONLY.  Used by tests/, the smoke check and the bench's CPU-baseline leg;
never by the product path.  Shares no code with the HIP library.

Definitions (restated from the pages; the derivation is in oracle.c's header):

* 1D causal long convolution -- "FlashFFTConv: Efficient Convolutions for Long Sequences with
  Tensor Cores" (abstract: the method computes exact FFT convolutions) and the Caracal abstract
  on the "RubiConv" page (causality from one-sided zero padding plus truncation):
      y[b,h,t] = v[b,h,t] * ( sum_{s<=t} k[h,t-s] x[b,h,s] + D[h] x[b,h,t] ),  x = q*u.
* 2D linear (non-circular) convolution with a centred, full-size kernel -- "Native
  Multi-Dimensional Subquadratic Operators via Input Dependent Long Convolutions" (abstract),
  for Hs x Ws images (halves rounded down):
      y[b,c,i,j] = sum_{a,e} k[c,a,e] u[b,c,i+Hs/2-a,j+Ws/2-e] + D[c] u[b,c,i,j].

Arrays are passed in their storage dtype: float32, float16, or bfloat16 carried as uint16 bit
patterns (the caller says which via ``dt``).  The C code widens them exactly to float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

DT_F32, DT_F16, DT_BF16 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (host code only)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-std=c11",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        vp, i64, dp, ip = ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.oracle_conv1d_rows.argtypes = [vp, vp, vp, vp, vp, ip, i64, i64, i64, vp, i64, dp, ip]
        lib.oracle_conv1d_points.argtypes = [vp, vp, vp, vp, vp, ip, i64, i64, i64, vp, i64, dp, ip]
        lib.oracle_conv1d_circ_rows.argtypes = [vp, vp, vp, dp, vp, ip, i64, i64, i64, i64, vp, i64,
                                                dp, ip]
        lib.oracle_conv1d_short_points.argtypes = [vp, vp, vp, vp, vp, ip, i64, i64, i64, i64, vp, i64,
                                                   dp, ip]
        lib.oracle_conv2d_points.argtypes = [vp, vp, vp, ip, i64, i64, i64, i64, vp, i64, dp, ip]
        lib.oracle_conv3d_points.argtypes = [vp, vp, vp, ip, i64, i64, i64, vp, i64, dp, ip]
        lib.oracle_ssm_rows.argtypes = [vp, vp, vp, dp, dp, vp, ip, i64, i64, i64, i64, vp, i64, dp, ip]
        lib.oracle_widen.argtypes = [vp, ip, i64, dp]
        lib.oracle_conv1d_bwd_rows.argtypes = [vp, vp, vp, vp, vp, vp, ip, i64, i64, i64, vp, i64,
                                               dp, dp, dp, ip]
        lib.oracle_conv1d_bwd_dk.argtypes = [vp, vp, vp, vp, ip, i64, i64, i64, vp, i64, dp, dp, ip]
        lib.oracle_conv1d_bwd_points.argtypes = [vp, vp, vp, vp, vp, vp, ip, i64, i64, i64, vp, i64,
                                                 dp, dp, dp, ip]
        lib.oracle_conv1d_bwd_dk_points.argtypes = [vp, vp, vp, vp, ip, i64, i64, i64, vp, i64, dp, ip]
        for f in (lib.oracle_conv1d_rows, lib.oracle_conv1d_points, lib.oracle_conv2d_points,
                  lib.oracle_conv1d_bwd_rows, lib.oracle_conv1d_bwd_dk):
            f.restype = ctypes.c_int
        lib.oracle_widen.restype = None
        _lib = lib
    return _lib


def _dt_of(a: np.ndarray, dt):
    if dt is not None:
        return dt
    if a.dtype == np.float32:
        return DT_F32
    if a.dtype == np.float16:
        return DT_F16
    raise ValueError("uint16 arrays are bfloat16 bit patterns: pass dt=DT_BF16 explicitly")


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def _storage(dt):
    return {DT_F32: np.float32, DT_F16: np.float16, DT_BF16: np.uint16}[dt]


def _threads(nthreads):
    if nthreads:
        return int(nthreads)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def widen(a: np.ndarray, dt=None) -> np.ndarray:
    """Exact float64 value of every element of a storage-dtype array (C widening)."""
    dt = _dt_of(a, dt)
    a = _c(a, _storage(dt))
    out = np.empty(a.size, np.float64)
    _load().oracle_widen(_ptr(a), dt, a.size, out.ctypes.data)
    return out.reshape(a.shape)


def conv1d_rows(u, k, D, rows, q=None, v=None, dt=None, nthreads=None):
    """Full output rows: returns float64 [len(rows), N] for rows = [(b,h), ...]."""
    dt = _dt_of(u, dt)
    st = _storage(dt)
    u, k, D, q, v = (_c(a, st) for a in (u, k, D, q, v))
    B, H, N = u.shape
    assert k.shape == (H, N) and D.shape == (H,)
    rows = np.ascontiguousarray(np.asarray(rows, np.int64).reshape(-1, 2))
    out = np.empty((rows.shape[0], N), np.float64)
    rc = _load().oracle_conv1d_rows(_ptr(u), _ptr(q), _ptr(v), _ptr(k), _ptr(D), dt, B, H, N,
                                    _ptr(rows), rows.shape[0], out.ctypes.data,
                                    _threads(nthreads))
    if rc:
        raise ValueError("oracle_conv1d_rows rejected its arguments")
    return out


def conv1d_points(u, k, D, pts, q=None, v=None, dt=None, nthreads=None):
    """Single outputs y[b,h,t] for pts = [(b,h,t), ...]; returns float64 [len(pts)]."""
    dt = _dt_of(u, dt)
    st = _storage(dt)
    u, k, D, q, v = (_c(a, st) for a in (u, k, D, q, v))
    B, H, N = u.shape
    pts = np.ascontiguousarray(np.asarray(pts, np.int64).reshape(-1, 3))
    out = np.empty(pts.shape[0], np.float64)
    rc = _load().oracle_conv1d_points(_ptr(u), _ptr(q), _ptr(v), _ptr(k), _ptr(D), dt, B, H, N,
                                      _ptr(pts), pts.shape[0], out.ctypes.data,
                                      _threads(nthreads))
    if rc:
        raise ValueError("oracle_conv1d_points rejected its arguments")
    return out


def conv1d_short_points(u, k, D, pts, q=None, v=None, dt=None, nthreads=None):
    """Single outputs y[b,h,t] with a short filter k [H, L] (zero beyond L taps; N may exceed L):
    the causal sum over the last L inputs (oracle.c).  Returns float64 [len(pts)]."""
    dt = _dt_of(u, dt)
    st = _storage(dt)
    u, k, D, q, v = (_c(a, st) for a in (u, k, D, q, v))
    B, H, N = u.shape
    L = k.shape[1]
    assert k.shape == (H, L) and D.shape == (H,)
    pts = np.ascontiguousarray(np.asarray(pts, np.int64).reshape(-1, 3))
    out = np.empty(pts.shape[0], np.float64)
    rc = _load().oracle_conv1d_short_points(_ptr(u), _ptr(q), _ptr(v), _ptr(k), _ptr(D), dt, B, H,
                                            N, L, _ptr(pts), pts.shape[0], out.ctypes.data,
                                            _threads(nthreads))
    if rc:
        raise ValueError("oracle_conv1d_short_points rejected its arguments")
    return out


def transform_length(N: int) -> int:
    """The transform length the method uses for N: the power of two M >= max(512, 2N)."""
    M = 512
    while M < 2 * N:
        M *= 2
    return M


def sparse_filter(k, keep, M=None, dt=None):
    """Frequency-sparse filter (FlashFFTConv abstract: skip blocks of the decomposition): the
    length-M DFT of the zero-padded filter k [H, N], kept only at frequencies f whose residue
    f mod R (R = M / 256, the blocks of the M = 256 R decomposition) is in `keep`, then inverse
    transformed.  `keep` must hold R - r with every r (else the filter would not be real).
    numpy's FFT serves as the DFT step.  Returns float64 [H, M]."""
    dt = _dt_of(k, dt)
    kk = widen(_c(k, _storage(dt)), dt).reshape(k.shape)
    H, N = kk.shape
    M = transform_length(N) if M is None else M
    R = M // 256
    keep = sorted(set(int(r) for r in keep))
    if any(r < 0 or r >= R for r in keep) or any((R - r) % R not in keep for r in keep):
        raise ValueError("keep must be a subset of range(R) closed under r -> (R - r) mod R")
    mask = np.isin(np.arange(M) % R, keep)
    pad = np.zeros((H, M))
    pad[:, :N] = kk
    return np.fft.ifft(np.fft.fft(pad, axis=1) * mask[None, :], axis=1).real


def conv1d_circ_rows(u, kS, D, rows, q=None, v=None, dt=None, nthreads=None):
    """Full rows of the circular convolution with a float64 filter kS [H, M] (M >= 2N), truncated
    to N (oracle.c).  Returns float64 [len(rows), N]."""
    dt = _dt_of(u, dt)
    st = _storage(dt)
    u, D, q, v = (_c(a, st) for a in (u, D, q, v))
    kS = np.ascontiguousarray(kS, np.float64)
    B, H, N = u.shape
    M = kS.shape[1]
    assert kS.shape == (H, M) and D.shape == (H,)
    rows = np.ascontiguousarray(np.asarray(rows, np.int64).reshape(-1, 2))
    out = np.empty((rows.shape[0], N), np.float64)
    rc = _load().oracle_conv1d_circ_rows(_ptr(u), _ptr(q), _ptr(v), kS.ctypes.data, _ptr(D), dt, B,
                                         H, N, M, _ptr(rows), rows.shape[0], out.ctypes.data,
                                         _threads(nthreads))
    if rc:
        raise ValueError("oracle_conv1d_circ_rows rejected its arguments")
    return out


def conv1d_bwd_rows(u, k, D, gy, rows, q=None, v=None, dt=None, nthreads=None):
    """Gradient rows of the causal convolution for rows = [(b,h), ...], given the output
    gradient gy [B,H,N]: returns float64 (du, dq, dv), each [len(rows), N] (dq is None without q,
    dv is None without v).  The chain rule on the plain definition, summed directly (oracle.c)."""
    dt = _dt_of(u, dt)
    st = _storage(dt)
    u, k, D, gy, q, v = (_c(a, st) for a in (u, k, D, gy, q, v))
    B, H, N = u.shape
    assert k.shape == (H, N) and D.shape == (H,) and gy.shape == u.shape
    rows = np.ascontiguousarray(np.asarray(rows, np.int64).reshape(-1, 2))
    du = np.empty((rows.shape[0], N), np.float64)
    dq = np.empty_like(du) if q is not None else None
    dv = np.empty_like(du) if v is not None else None
    rc = _load().oracle_conv1d_bwd_rows(_ptr(u), _ptr(q), _ptr(v), _ptr(k), _ptr(D), _ptr(gy), dt,
                                        B, H, N, _ptr(rows), rows.shape[0], du.ctypes.data,
                                        None if dq is None else dq.ctypes.data,
                                        None if dv is None else dv.ctypes.data, _threads(nthreads))
    if rc:
        raise ValueError("oracle_conv1d_bwd_rows rejected its arguments")
    return du, dq, dv


def conv1d_bwd_dk(u, gy, chans, q=None, v=None, dt=None, nthreads=None):
    """Filter and skip gradients for channels chans: returns float64 (dk [len(chans), N],
    dD [len(chans)]), dk[h,tau] = sum_b sum_t ds[b,h,t] x[b,h,t-tau] with ds = gy v, x = q u."""
    dt = _dt_of(u, dt)
    st = _storage(dt)
    u, gy, q, v = (_c(a, st) for a in (u, gy, q, v))
    B, H, N = u.shape
    chans = np.ascontiguousarray(np.asarray(chans, np.int64).reshape(-1))
    dk = np.empty((chans.shape[0], N), np.float64)
    dD = np.empty(chans.shape[0], np.float64)
    rc = _load().oracle_conv1d_bwd_dk(_ptr(u), _ptr(q), _ptr(v), _ptr(gy), dt, B, H, N, _ptr(chans),
                                      chans.shape[0], dk.ctypes.data, dD.ctypes.data,
                                      _threads(nthreads))
    if rc:
        raise ValueError("oracle_conv1d_bwd_dk rejected its arguments")
    return dk, dD


def conv1d_bwd_points(u, k, D, gy, pts, q=None, v=None, dt=None, nthreads=None):
    """The gradients du, dq, dv of conv1d_bwd_rows at single positions pts = [(b,h,t), ...],
    summed exactly as the row version sums them.  Returns float64 (du, dq, dv) of len(pts) each
    (dq None without q, dv None without v)."""
    dt = _dt_of(u, dt)
    st = _storage(dt)
    u, k, D, gy, q, v = (_c(a, st) for a in (u, k, D, gy, q, v))
    B, H, N = u.shape
    assert k.shape == (H, N) and D.shape == (H,) and gy.shape == u.shape
    pts = np.ascontiguousarray(np.asarray(pts, np.int64).reshape(-1, 3))
    du = np.empty(pts.shape[0], np.float64)
    dq = np.empty_like(du) if q is not None else None
    dv = np.empty_like(du) if v is not None else None
    rc = _load().oracle_conv1d_bwd_points(_ptr(u), _ptr(q), _ptr(v), _ptr(k), _ptr(D), _ptr(gy), dt, B, H,
                                          N, _ptr(pts), pts.shape[0], du.ctypes.data,
                                          None if dq is None else dq.ctypes.data,
                                          None if dv is None else dv.ctypes.data, _threads(nthreads))
    if rc:
        raise ValueError("oracle_conv1d_bwd_points rejected its arguments")
    return du, dq, dv


def conv1d_bwd_dk_points(u, gy, pts, q=None, v=None, dt=None, nthreads=None):
    """dk[h, tau] of conv1d_bwd_dk at pairs pts = [(h, tau), ...], summed exactly as the channel
    version sums them.  Returns float64 [len(pts)]."""
    dt = _dt_of(u, dt)
    st = _storage(dt)
    u, gy, q, v = (_c(a, st) for a in (u, gy, q, v))
    B, H, N = u.shape
    pts = np.ascontiguousarray(np.asarray(pts, np.int64).reshape(-1, 2))
    dk = np.empty(pts.shape[0], np.float64)
    rc = _load().oracle_conv1d_bwd_dk_points(_ptr(u), _ptr(q), _ptr(v), _ptr(gy), dt, B, H, N, _ptr(pts),
                                             pts.shape[0], dk.ctypes.data, _threads(nthreads))
    if rc:
        raise ValueError("oracle_conv1d_bwd_dk_points rejected its arguments")
    return dk


def _short_as_full(k, N):
    """A short filter k [H, L] (storage dtype) as the N-tap filter it acts as on length-N rows:
    its first min(L, N) taps, then zeros (taps at lags >= N never meet an input)."""
    k = np.asarray(k)
    H, L = k.shape
    kN = np.zeros((H, N), k.dtype)  # zero bits are 0.0 in every storage type
    m = min(L, N)
    kN[:, :m] = k[:, :m]
    return kN


def conv1d_short_bwd_rows(u, k, D, gy, rows, q=None, v=None, dt=None, nthreads=None):
    """Gradient rows (du, dq, dv) of the convolution with a short filter k [H, L] (the partial
    convolution of the FlashFFTConv abstract): the chain rule on the causal sum over the last L
    inputs, i.e. conv1d_bwd_rows with k taken as the N-tap filter it acts as."""
    N = np.asarray(u).shape[2]
    return conv1d_bwd_rows(u, _short_as_full(k, N), D, gy, rows, q=q, v=v, dt=_dt_of(u, dt), nthreads=nthreads)


def conv1d_short_bwd_points(u, k, D, gy, pts, q=None, v=None, dt=None, nthreads=None):
    """conv1d_short_bwd_rows at single positions pts = [(b,h,t), ...]."""
    N = np.asarray(u).shape[2]
    return conv1d_bwd_points(u, _short_as_full(k, N), D, gy, pts, q=q, v=v, dt=_dt_of(u, dt), nthreads=nthreads)


def conv1d_short_bwd_dk(u, gy, chans, L, q=None, v=None, dt=None, nthreads=None):
    """Filter and skip gradients of the short-filter convolution: (dk [len(chans), L], dD).  The
    filter enters only through its taps, so dk[h, tau] is the correlation of conv1d_bwd_dk at
    lag tau < min(L, N); lags tau >= N have no pair of positions and are zero."""
    N = np.asarray(u).shape[2]
    dk, dD = conv1d_bwd_dk(u, gy, chans, q=q, v=v, dt=_dt_of(u, dt), nthreads=nthreads)
    out = np.zeros((dk.shape[0], L), np.float64)
    m = min(L, N)
    out[:, :m] = dk[:, :m]
    return out, dD


def conv1d_short_bwd_dk_points(u, gy, pts, L, q=None, v=None, dt=None, nthreads=None):
    """dk[h, tau] of conv1d_short_bwd_dk at pairs pts = [(h, tau), ...] with tau < L."""
    N = np.asarray(u).shape[2]
    pts = np.asarray(pts, np.int64).reshape(-1, 2)
    assert np.all(pts[:, 1] < L)
    out = np.zeros(pts.shape[0], np.float64)
    inside = pts[:, 1] < N
    if np.any(inside):
        out[inside] = conv1d_bwd_dk_points(u, gy, pts[inside], q=q, v=v, dt=_dt_of(u, dt), nthreads=nthreads)
    return out


def conv2d_points(u, k, D, pts, dt=None, nthreads=None):
    """Direct 2D sums y[b,c,i,j] for pts = [(b,c,i,j), ...] (u [B,C,Hs,Ws], k [C,Hs,Ws], centre
    tap (Hs//2, Ws//2)); returns float64 [len(pts)]."""
    dt = _dt_of(u, dt)
    st = _storage(dt)
    u, k, D = (_c(a, st) for a in (u, k, D))
    B, C, Hs, Ws = u.shape
    assert k.shape == (C, Hs, Ws) and D.shape == (C,)
    pts = np.ascontiguousarray(np.asarray(pts, np.int64).reshape(-1, 4))
    out = np.empty(pts.shape[0], np.float64)
    rc = _load().oracle_conv2d_points(_ptr(u), _ptr(k), _ptr(D), dt, B, C, Hs, Ws, _ptr(pts),
                                      pts.shape[0], out.ctypes.data, _threads(nthreads))
    if rc:
        raise ValueError("oracle_conv2d_points rejected its arguments")
    return out


def conv2d_bwd(u, k, D, gy, images=None, chans=None, dt=None):
    """Gradients of the centred 2D convolution (conv2d_points' definition) given gy = dL/dy
    [B,C,Hs,Ws], in float64 from the exact values of the storage-dtype inputs:
        du[b,c,m,n] = sum_{i,j} gy[b,c,i,j] k[c, i+Hs/2-m, j+Ws/2-n] + D[c] gy[b,c,m,n]
        dk[c,a,e]   = sum_{b,i,j} gy[b,c,i,j] u[b,c, i+Hs/2-a, j+Ws/2-e]
        dD[c]       = sum_{b,i,j} gy[b,c,i,j] u[b,c,i,j]
    (halves rounded down, u and k zero outside their extent).  With G = gy placed at rows
    [Hs/2, Hs/2+Hs) and columns [Ws/2, Ws/2+Ws) of a (2Hs-1) x (2Ws-1) zero grid, du = the valid
    correlation of G with k plus D gy, and dk = the batch sum of the valid correlations of G with
    u (scipy.signal.correlate, float64).  images: (b, c) pairs for du (default all); chans: the
    channels for dk and dD (default all).  Returns (du [len(images),Hs,Ws], dk [len(chans),Hs,Ws],
    dD [len(chans)])."""
    from scipy.signal import correlate
    dt = _dt_of(u, dt)
    u, k, D, gy = (widen(a, dt) for a in (u, k, D, gy))
    B, C, Hs, Ws = u.shape
    assert k.shape == (C, Hs, Ws) and D.shape == (C,) and gy.shape == u.shape
    h, w = Hs // 2, Ws // 2
    if images is None:
        images = [(b, c) for b in range(B) for c in range(C)]
    if chans is None:
        chans = list(range(C))

    def grid(b, c):
        G = np.zeros((2 * Hs - 1, 2 * Ws - 1))
        G[h:h + Hs, w:w + Ws] = gy[b, c]
        return G

    du = np.stack([correlate(grid(b, c), k[c], mode="valid") + D[c] * gy[b, c] for b, c in images]) \
        if len(images) else np.zeros((0, Hs, Ws))
    dk = np.stack([sum(correlate(grid(b, c), u[b, c], mode="valid") for b in range(B)) for c in chans]) \
        if len(chans) else np.zeros((0, Hs, Ws))
    dD = np.asarray([float(np.sum(gy[:, c] * u[:, c])) for c in chans])
    return du, dk, dD


def ssm_kernel(lam, W, N):
    """The filter of a diagonal state-space model: k[h, t] = Re sum_n W[h, n] lam[h, n]^t for
    t < N (lam, W complex [H, NS]), by repeated multiplication in float64 complex."""
    lam = np.asarray(lam, np.complex128)
    W = np.asarray(W, np.complex128)
    H, NS = lam.shape
    k = np.empty((H, N))
    p = np.ones((H, NS), np.complex128)
    for t in range(N):
        k[:, t] = (W * p).sum(axis=1).real
        p = p * lam
    return k


def ssm_rows(u, lam, W, D, rows, q=None, v=None, dt=None, nthreads=None):
    """Full output rows of the convolution with the state-space filter (lam, W complex [H, NS]),
    evaluated by the state recurrence (oracle.c).  Returns float64 [len(rows), N]."""
    dt = _dt_of(u, dt)
    st = _storage(dt)
    u, D, q, v = (_c(a, st) for a in (u, D, q, v))
    lam = np.ascontiguousarray(np.asarray(lam, np.complex128))
    W = np.ascontiguousarray(np.asarray(W, np.complex128))
    B, H, N = u.shape
    NS = lam.shape[1]
    assert lam.shape == (H, NS) and W.shape == (H, NS) and D.shape == (H,)
    rows = np.ascontiguousarray(np.asarray(rows, np.int64).reshape(-1, 2))
    out = np.empty((rows.shape[0], N), np.float64)
    rc = _load().oracle_ssm_rows(_ptr(u), _ptr(q), _ptr(v), lam.ctypes.data, W.ctypes.data, _ptr(D),
                                 dt, B, H, N, NS, _ptr(rows), rows.shape[0], out.ctypes.data,
                                 _threads(nthreads))
    if rc:
        raise ValueError("oracle_ssm_rows rejected its arguments")
    return out


def conv3d_points(u, k, D, pts, dt=None, nthreads=None):
    """Direct 3D sums y[b,c,i,j,l] for pts = [(b,c,i,j,l), ...] (u [B,C,S,S,S], k [C,S,S,S],
    centred kernel, cropped to the window, plus D u); returns float64 [len(pts)]."""
    dt = _dt_of(u, dt)
    st = _storage(dt)
    u, k, D = (_c(a, st) for a in (u, k, D))
    B, C, S = u.shape[:3]
    assert u.shape == (B, C, S, S, S) and k.shape == (C, S, S, S) and D.shape == (C,)
    pts = np.ascontiguousarray(np.asarray(pts, np.int64).reshape(-1, 5))
    out = np.empty(pts.shape[0], np.float64)
    rc = _load().oracle_conv3d_points(_ptr(u), _ptr(k), _ptr(D), dt, B, C, S, _ptr(pts),
                                      pts.shape[0], out.ctypes.data, _threads(nthreads))
    if rc:
        raise ValueError("oracle_conv3d_points rejected its arguments")
    return out


def _dft_matrix(P: int, rows, cols, sign: int) -> np.ndarray:
    """exp(sign * 2*pi*i * (r*c mod P) / P) with the exponent reduced exactly in integers."""
    r = np.asarray(rows, np.int64)[:, None]
    c = np.asarray(cols, np.int64)[None, :]
    red = (r * c) % P
    ang = (2.0 * np.pi / P) * red.astype(np.float64)
    return np.cos(ang) + sign * 1j * np.sin(ang)


def conv2d_dft(u, k, D, images, dt=None, P=None):
    """Naive separable-DFT 2D oracle (independent of the direct sums).

    For each image (b,c) of Hs x Ws: zero pad u and k to Ph x Pw (Ph >= 2Hs-1, Pw >= 2Ws-1,
    default 2Hs x 2Ws, so the product of spectra is a *linear* convolution), multiply the 2D
    DFTs, invert only the Hs x Ws window of rows [Hs/2, Hs/2+Hs) and columns [Ws/2, Ws/2+Ws)
    (halves rounded down) and add D*u.  The DFTs are explicit matrices applied with matmul; no
    FFT routine is involved.  P = (Ph, Pw) or one side for both.  Returns float64
    [len(images), Hs, Ws].
    """
    dt = _dt_of(u, dt)
    uw = widen(u, dt)
    kw = widen(k, dt)
    Dw = widen(D, dt)
    B, C, Hs, Ws = uw.shape
    Ph, Pw = (P, P) if isinstance(P, int) else (P or (2 * Hs, 2 * Ws))
    assert Ph >= 2 * Hs - 1 and Pw >= 2 * Ws - 1
    Fh = _dft_matrix(Ph, range(Ph), range(Hs), -1)                        # [Ph, Hs] forward
    Fw = _dft_matrix(Pw, range(Pw), range(Ws), -1)                        # [Pw, Ws]
    Gh = _dft_matrix(Ph, range(Hs // 2, Hs // 2 + Hs), range(Ph), +1)     # [Hs, Ph] inverse, crop
    Gw = _dft_matrix(Pw, range(Ws // 2, Ws // 2 + Ws), range(Pw), +1)     # [Ws, Pw]
    out = []
    kf_cache = {}
    for (b, c) in np.asarray(images, np.int64).reshape(-1, 2):
        b, c = int(b), int(c)
        if c not in kf_cache:
            kf_cache[c] = Fh @ kw[c] @ Fw.T
        U = Fh @ uw[b, c] @ Fw.T
        Y = (Gh @ (U * kf_cache[c]) @ Gw.T) / (Ph * Pw)
        out.append(Y.real + Dw[c] * uw[b, c])
    return np.stack(out) if out else np.zeros((0, Hs, Ws))


# --------------------------------------------------------------------------------------------
# Small-case references used to pin the C oracle (pure Python / explicit matrices).
# --------------------------------------------------------------------------------------------

def conv1d_toeplitz(x: np.ndarray, k: np.ndarray, d: float) -> np.ndarray:
    """y = T x + d x with T[t,s] = k[t-s] for s <= t (explicit lower-triangular Toeplitz)."""
    N = x.shape[-1]
    T = np.zeros((N, N), np.float64)
    for t in range(N):
        T[t, : t + 1] = k[t::-1]
    return T @ x + d * x


def conv1d_python_int(x, k, d):
    """Exact integer causal convolution with Python ints (for N <= 64 brute force)."""
    N = len(x)
    return [sum(int(k[t - s]) * int(x[s]) for s in range(t + 1)) + int(d) * int(x[t])
            for t in range(N)]

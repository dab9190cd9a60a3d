"""float64 oracle of the learned-Butterfly long convolution.

TEST INFRASTRUCTURE ONLY.  Used by tests/; never by the product path.  Shares no code with the
HIP library.

Source: "Simple Hardware-Efficient Long Convolutions for Sequence Modeling", abstract: the
coefficients of the Butterfly decomposition of the FFT can be learned, at the runtime of the
fixed decomposition.  The page gives no formula; the reading used here (listed with the other
readings of the pages in the design notes):

* The decomposition is the three-digit split of an M-point transform, M = 256 R,
      n = 256 n1 + 16 n2 + n3,      f = k1 + R k2 + 16 R k3,
  whose dense factor blocks are the free parameters:
      forward  X[f] = sum_{n3} A3[k1,k3,n3] w256^{n3 k2} sum_{n2} A2[k1,k2,n2] sum_{n1} A1[k1,n1] x[n]
      inverse  z[n] = sum_{k1} B3[n1,k1] sum_{k2} B2[k1,n2,k2] conj(w256^{n3 k2})
                            sum_{k3} B1[k1,n3,k3] Z[f]
  with w256 = exp(-2 pi i / 256) fixed.  The DFT's own blocks (dft_blocks) make the forward map
  the DFT and the inverse map M times the inverse DFT.
* The convolution keeps the shape of the FFT one: x = q u and the filter k are zero-padded to
  M = transform_length(N), K = forward(k) / M, and
      y = v * ( Re(inverse(K * forward(x)))[:N] + D x ).
  With dft_blocks this is the causal convolution (oracle.conv1d_rows).

Each step is a contraction over one digit (numpy einsum), in the order above.
"""
from __future__ import annotations

import numpy as np

from .oracle import transform_length, widen


def _radix(M: int) -> int:
    if M % 256 or M < 512:
        raise ValueError("M must be 256 R with R >= 2")
    return M // 256


def _w256() -> np.ndarray:
    """T[k2, n3] = exp(-2 pi i k2 n3 / 256), the fixed twiddle."""
    e = np.outer(np.arange(16), np.arange(16)) % 256
    return np.exp(-2j * np.pi * e / 256.0)


def dft_blocks(M: int) -> dict:
    """The DFT's factor blocks for M = 256 R (exponents reduced exactly in integers)."""
    R = _radix(M)
    k1 = np.arange(R)[:, None, None]
    a = np.arange(16)

    def w(e, P):
        return np.exp(-2j * np.pi * (np.asarray(e) % P) / P)

    A1 = w(np.outer(np.arange(R), np.arange(R)), R)                              # [k1, n1]
    A2 = w(a[None, None, :] * (k1 + R * a[None, :, None]), 16 * R)                # [k1, k2, n2]
    A3 = w(a[None, None, :] * (k1 + 16 * R * a[None, :, None]), M)                # [k1, k3, n3]
    return {"A1": A1, "A2": A2, "A3": A3,
            "B1": np.conj(np.swapaxes(A3, 1, 2)),                                 # [k1, n3, k3]
            "B2": np.conj(np.swapaxes(A2, 1, 2)),                                 # [k1, n2, k2]
            "B3": np.conj(A1.T)}                                                  # [n1, k1]


def unpack_blocks(flat: np.ndarray, M: int) -> dict:
    """Blocks from the flat complex array of the C ABI: A1 [R][R], A2, A3, B1, B2 [R][16][16],
    B3 [R][R], back to back."""
    R = _radix(M)
    flat = np.asarray(flat).astype(np.complex128).ravel()
    sizes = [R * R, 256 * R, 256 * R, 256 * R, 256 * R, R * R]
    if flat.size != sum(sizes):
        raise ValueError("expected %d complex values" % sum(sizes))
    out, o = {}, 0
    for name, n in zip(("A1", "A2", "A3", "B1", "B2", "B3"), sizes):
        part = flat[o:o + n]
        out[name] = part.reshape(R, R) if n == R * R else part.reshape(R, 16, 16)
        o += n
    return out


def forward(x: np.ndarray, bl: dict) -> np.ndarray:
    """X[..., f] (natural f) of x[..., n] (natural n), M = x.shape[-1]."""
    M = x.shape[-1]
    R = _radix(M)
    xs = np.asarray(x, dtype=np.complex128).reshape(x.shape[:-1] + (R, 16, 16))        # [n1, n2, n3]
    a = np.einsum("kn,...nbc->...kbc", bl["A1"], xs)                                  # [k1, n2, n3]
    b = np.einsum("kpn,...knc->...kpc", bl["A2"], a)                                  # [k1, k2, n3]
    c = b * _w256()                                                                   # w256^{n3 k2}
    X = np.einsum("kqc,...kpc->...kpq", bl["A3"], c)                                  # [k1, k2, k3]
    # f = k1 + R k2 + 16 R k3: k3 slowest
    return np.moveaxis(X, (-3, -2, -1), (-1, -2, -3)).reshape(x.shape[:-1] + (M,))


def inverse(Z: np.ndarray, bl: dict) -> np.ndarray:
    """z[..., n] (natural n) of Z[..., f] (natural f)."""
    M = Z.shape[-1]
    R = _radix(M)
    Zr = np.moveaxis(np.asarray(Z, dtype=np.complex128).reshape(Z.shape[:-1] + (16, 16, R)),
                     (-3, -2, -1), (-1, -2, -3))                                      # [k1, k2, k3]
    s = np.einsum("kcq,...kpq->...kpc", bl["B1"], Zr)                                 # [k1, k2, n3]
    s = s * np.conj(_w256())
    r = np.einsum("knp,...kpc->...knc", bl["B2"], s)                                  # [k1, n2, n3]
    z = np.einsum("mk,...kbc->...mbc", bl["B3"], r)                                   # [n1, n2, n3]
    return z.reshape(Z.shape[:-1] + (M,))


def dense(bl: dict, M: int):
    """The forward and inverse maps as dense M x M matrices, entry by entry: every (f, n) pair
    has one path through the factors,
        T[f, n] = A3[k1,k3,n3] w256^{n3 k2} A2[k1,k2,n2] A1[k1,n1]
        S[n, f] = B3[n1,k1] B2[k1,n2,k2] conj(w256^{n3 k2}) B1[k1,n3,k3]."""
    R = _radix(M)
    f = np.arange(M)
    n = np.arange(M)
    k1, k2, k3 = f % R, (f // R) % 16, f // (16 * R)
    n1, n2, n3 = n // 256, (n // 16) % 16, n % 16
    tw = _w256()
    T = (bl["A3"][k1[:, None], k3[:, None], n3[None, :]] * tw[k2[:, None], n3[None, :]]
         * bl["A2"][k1[:, None], k2[:, None], n2[None, :]] * bl["A1"][k1[:, None], n1[None, :]])
    S = (bl["B3"][n1[:, None], k1[None, :]] * bl["B2"][k1[None, :], n2[:, None], k2[None, :]]
         * np.conj(tw[k2[None, :], n3[:, None]]) * bl["B1"][k1[None, :], n3[:, None], k3[None, :]])
    return T, S


def butterfly_conv(u, k, D, blocks, q=None, v=None, dt=None) -> np.ndarray:
    """y[b,h,t] = v * ( Re(inverse(K[h] * forward(x[b,h])))[t] + D[h] x[b,h,t] ), t < N, with
    x = q u, both zero-padded to M = transform_length(N), K = forward(k) / M.  ``blocks``: a dict
    (dft_blocks) or the flat complex array of the C ABI.  Inputs in their storage dtype (``dt``
    as in oracle.conv1d_rows); returns float64 [B, H, N]."""
    u = widen(u, dt)
    k = widen(k, dt)
    D = widen(D, dt)
    B, H, N = u.shape
    M = transform_length(N)
    bl = blocks if isinstance(blocks, dict) else unpack_blocks(blocks, M)
    x = u * widen(q, dt) if q is not None else u
    xp = np.zeros((B, H, M))
    xp[..., :N] = x
    kp = np.zeros((H, M))
    kp[:, :N] = k
    K = forward(kp, bl) / M
    z = inverse(forward(xp, bl) * K[None], bl)
    y = z.real[..., :N] + D[None, :, None] * x
    if v is not None:
        y = y * widen(v, dt)
    return y

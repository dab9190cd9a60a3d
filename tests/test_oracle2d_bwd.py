"""Pins for the 2D gradient oracle (oracle.conv2d_bwd), CPU only.

The centred 2D convolution of the HyenaND abstract is linear in u, in k and in D separately, so
every gradient element is the loss <dy, y> of a forward with one operand set to a unit vector:
    du[b,c,m,n] = <dy, y(u = e_bcmn)>,  dk[c,a,e] = <dy, y(k = e_cae, D = 0)>,  dD[c] = <dy, y(k = 0, D = e_c)>.
The forward is oracle.conv2d_points (direct sums, pinned in the 2D oracle tests), independent of
the correlations the gradient oracle uses, so this brute force checks it element by element on
square, rectangular and odd shapes (the centre tap sits at the rounded-down halves; an off-by-one
in either half, a transposed kernel or a missing skip term fails).  float32 inputs, float64 sums.
"""
import numpy as np
import pytest

import oracle


def _draw(B, C, Hs, Ws, seed):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    return f(B, C, Hs, Ws), f(C, Hs, Ws), f(C), f(B, C, Hs, Ws)


def _loss(u, k, D, dy):
    B, C, Hs, Ws = u.shape
    pts = [(b, c, i, j) for b in range(B) for c in range(C) for i in range(Hs) for j in range(Ws)]
    y = oracle.conv2d_points(u, k, D, pts, nthreads=1)
    return float(np.dot(dy.reshape(-1).astype(np.float64), y))


def _unit(shape, idx):
    e = np.zeros(int(np.prod(shape)), np.float32)
    e[idx] = 1.0
    return e.reshape(shape)


@pytest.mark.parametrize("B,C,Hs,Ws", [(2, 2, 4, 4), (1, 2, 3, 5), (2, 1, 5, 2), (1, 1, 6, 7)])
def test_conv2d_bwd_oracle_brute_force(B, C, Hs, Ws):
    u, k, D, dy = _draw(B, C, Hs, Ws, seed=10 * Hs + Ws + B)
    du, dk, dD = oracle.conv2d_bwd(u, k, D, dy)
    bu = np.array([_loss(_unit(u.shape, i), k, D, dy) for i in range(u.size)]).reshape(B * C, Hs, Ws)
    zD = np.zeros_like(D)
    bk = np.array([_loss(u, _unit(k.shape, i), zD, dy) for i in range(k.size)]).reshape(C, Hs, Ws)
    bD = np.array([_loss(u, np.zeros_like(k), _unit(D.shape, c), dy) for c in range(C)])
    tol = lambda r: 1e-10 * max(1.0, float(np.max(np.abs(r))))
    assert np.max(np.abs(du - bu)) <= tol(bu)
    assert np.max(np.abs(dk - bk)) <= tol(bk)
    assert np.max(np.abs(dD - bD)) <= tol(bD)


def test_conv2d_bwd_subsets_match_full():
    """images / chans select rows of the full result."""
    u, k, D, dy = _draw(3, 2, 5, 6, seed=3)
    du, dk, dD = oracle.conv2d_bwd(u, k, D, dy)
    du2, dk2, dD2 = oracle.conv2d_bwd(u, k, D, dy, images=[(2, 1), (0, 0)], chans=[1])
    assert np.array_equal(du2[0], du[2 * 2 + 1]) and np.array_equal(du2[1], du[0])
    assert np.array_equal(dk2[0], dk[1]) and dD2[0] == dD[1]


def test_conv2d_bwd_planted_transpose_fails():
    """A kernel read transposed (k[c, e, a]) changes du on a non-symmetric kernel: the brute force
    sees the difference."""
    u, k, D, dy = _draw(1, 1, 4, 4, seed=5)
    du, _, _ = oracle.conv2d_bwd(u, k, D, dy)
    du_t, _, _ = oracle.conv2d_bwd(u, np.ascontiguousarray(k.transpose(0, 2, 1)), D, dy)
    assert np.max(np.abs(du - du_t)) > 1e-3

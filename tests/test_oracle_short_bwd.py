"""Pins for the short-filter gradient oracle (oracle.conv1d_short_bwd_*), CPU only.

The partial convolution of the FlashFFTConv abstract is linear in each of u, q, v, k and D when
the others are held fixed, so every gradient element is the loss <dy, y> of the forward with one
operand replaced by a unit vector:
    du[b,h,s] = <dy, y(u = e_bhs)>,   dq[b,h,s] = <dy, y(q = e_bhs)>,
    dv = dy (.) y(v = 1),   dk[h,tau] = <dy, y(k = e_h,tau, D = 0)>,   dD[h] = <dy, y(k = 0, D = e_h)>.
Each forward here is oracle.conv1d_short_points (pinned on its own in test_oracle_short.py), so
this brute force checks the gradient oracle element by element: a dropped or extra tap, a lag
past N that is not zero, a reversed filter or a swapped gate fails it.  float32 inputs, float64
sums: agreement to rounding order (1e-12 relative).
"""
import numpy as np
import pytest

import oracle


def _draw(B, H, N, L, seed):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    return f(B, H, N), f(B, H, N), f(B, H, N), f(H, L), f(H), f(B, H, N)


def _y(u, k, D, q, v):
    B, H, N = u.shape
    pts = [(b, h, t) for b in range(B) for h in range(H) for t in range(N)]
    return oracle.conv1d_short_points(u, k, D, pts, q=q, v=v, nthreads=1).reshape(B, H, N)


def _brute(u, q, v, k, D, dy):
    B, H, N = u.shape
    L = k.shape[1]
    loss = lambda **kw: float(np.sum(dy.astype(np.float64) * _y(**{"u": u, "k": k, "D": D, "q": q, "v": v, **kw})))
    unit = lambda shape, idx: np.where(np.arange(np.prod(shape)).reshape(shape) == idx, 1.0, 0.0).astype(np.float32)
    du = np.array([loss(u=unit(u.shape, i)) for i in range(u.size)]).reshape(u.shape)
    dq = None if q is None else np.array([loss(q=unit(u.shape, i)) for i in range(u.size)]).reshape(u.shape)
    dv = None if v is None else dy.astype(np.float64) * _y(u, k, D, q, None)
    zD = np.zeros_like(D)
    dk = np.array([loss(k=unit(k.shape, i), D=zD) for i in range(k.size)]).reshape(H, L)
    dD = np.array([loss(k=np.zeros_like(k), D=unit(D.shape, h)) for h in range(H)])
    return du, dq, dv, dk, dD


def _close(a, b):
    scale = max(1.0, float(np.max(np.abs(b))))
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) <= 1e-12 * scale * 64


@pytest.mark.parametrize("B,H,N,L,gates", [
    (2, 2, 20, 8, "qv"),     # N > L
    (1, 2, 12, 32, "qv"),    # L > N: lags >= N must be zero
    (2, 1, 16, 16, ""),      # L = N, no gates
    (3, 1, 10, 4, "q"),
])
def test_short_bwd_oracle_brute_force(B, H, N, L, gates):
    u, q, v, k, D, dy = _draw(B, H, N, L, seed=B * 100 + N + L)
    q = q if "q" in gates else None
    v = v if "v" in gates else None
    du, dq, dv, dk, dD = _brute(u, q, v, k, D, dy)
    rows = [(b, h) for b in range(B) for h in range(H)]
    o_du, o_dq, o_dv = oracle.conv1d_short_bwd_rows(u, k, D, dy, rows, q=q, v=v, nthreads=1)
    assert _close(o_du.reshape(B, H, N), du)
    if q is None:
        assert o_dq is None
    else:
        assert _close(o_dq.reshape(B, H, N), dq)
    if v is None:
        assert o_dv is None
    else:
        assert _close(o_dv.reshape(B, H, N), dv)
    o_dk, o_dD = oracle.conv1d_short_bwd_dk(u, dy, list(range(H)), L, q=q, v=v, nthreads=1)
    assert o_dk.shape == (H, L)
    assert _close(o_dk, dk) and _close(o_dD, dD)
    if L > N:
        assert np.all(o_dk[:, N:] == 0.0)


def test_short_bwd_points_match_rows():
    """The point versions return the row versions' values bit for bit (same sums)."""
    B, H, N, L = 2, 3, 40, 16
    u, q, v, k, D, dy = _draw(B, H, N, L, seed=5)
    rows = [(b, h) for b in range(B) for h in range(H)]
    r_du, r_dq, r_dv = oracle.conv1d_short_bwd_rows(u, k, D, dy, rows, q=q, v=v, nthreads=1)
    pts = [(b, h, t) for b in range(B) for h in range(H) for t in range(N)]
    p_du, p_dq, p_dv = oracle.conv1d_short_bwd_points(u, k, D, dy, pts, q=q, v=v, nthreads=1)
    assert np.array_equal(p_du, r_du.reshape(-1)) and np.array_equal(p_dq, r_dq.reshape(-1))
    assert np.array_equal(p_dv, r_dv.reshape(-1))
    r_dk, _ = oracle.conv1d_short_bwd_dk(u, dy, list(range(H)), L, q=q, v=v, nthreads=1)
    kp = [(h, t) for h in range(H) for t in range(L)]
    assert np.array_equal(oracle.conv1d_short_bwd_dk_points(u, dy, kp, L, q=q, v=v, nthreads=1), r_dk.reshape(-1))


def test_short_bwd_planted_mistake_fails():
    """A gradient oracle that forgot to cut the filter at L (used taps past L on the zero-extended
    row) would still pass a test that draws k only L long; this one plants a tap past L into the
    forward and checks that the brute force sees it."""
    B, H, N, L = 1, 1, 16, 4
    u, q, v, k, D, dy = _draw(B, H, N, L, seed=9)
    du, _, _, _, _ = _brute(u, None, None, k, D, dy)
    k_long = np.concatenate([k, np.ones((H, 1), np.float32)], 1)   # one tap too many
    wrong, _, _ = oracle.conv1d_short_bwd_rows(u, k_long, D, dy, [(0, 0)], nthreads=1)
    assert not _close(wrong.reshape(B, H, N), du)

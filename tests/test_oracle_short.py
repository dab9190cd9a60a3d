"""Pins for the short-filter oracle (oracle.conv1d_short_points), CPU only.

A filter of L taps acting on N positions is the causal convolution with the filter zero beyond
its length ("partial convolutions", FlashFFTConv abstract).  Pinned by: agreement with the
full-length oracle on the zero-extended filter (L <= N) and on the truncated filter (L > N),
numpy.convolve, a delta input that returns the filter and then zeros, and exact integer
arithmetic.  Planted mistakes in the summation window (one tap too many, one too few, a
reversed filter, a dropped skip term) each fail a pin.
"""
import numpy as np
import pytest

import oracle


def _draw(B, H, N, L, seed):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    return f(B, H, N), f(B, H, N), f(B, H, N), f(H, L), f(H)


def all_pts(B, H, N):
    return [(b, h, t) for b in range(B) for h in range(H) for t in range(N)]


def short_numpy(u, k, D, pts, q=None, v=None, mutant=None):
    """Direct window sums in numpy, optionally with one planted mistake."""
    u, k, D = (np.asarray(a, np.float64) for a in (u, k, D))
    L = k.shape[1]
    x = u * (np.asarray(q, np.float64) if q is not None else 1.0)
    out = []
    for b, h, t in pts:
        kk = k[h][::-1] if mutant == "reversed" else k[h]
        lo = {"one_more": t - L, "one_less": t - L + 2}.get(mutant, t - L + 1)
        acc = sum(kk[t - s] * x[b, h, s] for s in range(max(0, lo), t + 1) if t - s < L)
        if mutant == "one_more" and t - L >= 0:
            acc += kk[L - 1] * x[b, h, t - L]      # an extra tap outside the filter
        if mutant != "no_skip":
            acc += D[h] * x[b, h, t]
        if v is not None:
            acc *= float(v[b, h, t])
        out.append(acc)
    return np.asarray(out)


def pin_zero_extended(fn):
    """Equals the full-length oracle with the filter zero-extended (L < N) or cut (L > N)."""
    ok = True
    for (N, L, seed) in ((40, 7, 1), (24, 24, 2), (16, 30, 3)):
        u, q, v, k, D = _draw(2, 2, N, L, seed)
        kz = np.zeros((2, N), np.float32)
        kz[:, :min(L, N)] = k[:, :min(L, N)]
        pts = all_pts(2, 2, N)
        ref = oracle.conv1d_points(u, kz, D, pts, q=q, v=v)
        ok &= np.allclose(fn(u, k, D, pts, q, v), ref, rtol=1e-12, atol=1e-12)
    return ok


def pin_numpy_convolve(fn):
    u, _, _, k, D = _draw(1, 1, 64, 9, 5)
    pts = all_pts(1, 1, 64)
    x = u[0, 0].astype(np.float64)
    ref = np.convolve(x, k[0].astype(np.float64))[:64] + float(D[0]) * x
    return np.allclose(fn(u, k, D, pts, None, None), ref, rtol=1e-12, atol=1e-12)


def pin_delta(fn):
    """u = e_0, no gates: the output is the filter, then zeros; D adds at t = 0."""
    N, L = 20, 6
    u = np.zeros((1, 1, N), np.float32)
    u[0, 0, 0] = 1
    k = np.arange(1, L + 1, dtype=np.float32)[None]
    D = np.asarray([0.5], np.float32)
    want = np.zeros(N)
    want[:L] = k[0]
    want[0] += 0.5
    return np.array_equal(fn(u, k, D, all_pts(1, 1, N), None, None), want)


def pin_integer(fn):
    rng = np.random.default_rng(9)
    N, L = 30, 5
    I = lambda *s: rng.integers(-4, 5, s).astype(np.float32)
    u, q, v, k, D = I(1, 1, N), I(1, 1, N), I(1, 1, N), I(1, L), I(1)
    x = [int(q[0, 0, s]) * int(u[0, 0, s]) for s in range(N)]
    want = [int(v[0, 0, t]) * (sum(int(k[0, t - s]) * x[s] for s in range(max(0, t - L + 1), t + 1))
                               + int(D[0]) * x[t]) for t in range(N)]
    return np.array_equal(fn(u, k, D, all_pts(1, 1, N), q, v), np.asarray(want, np.float64))


PINS = [pin_zero_extended, pin_numpy_convolve, pin_delta, pin_integer]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_short_oracle_passes_pins(pin):
    assert pin(lambda u, k, D, pts, q, v: oracle.conv1d_short_points(u, k, D, pts, q=q, v=v))


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_numpy_window_sum_passes_pins(pin):
    assert pin(lambda u, k, D, pts, q, v: short_numpy(u, k, D, pts, q, v))


@pytest.mark.parametrize("mutant", ["one_more", "one_less", "reversed", "no_skip"])
def test_planted_window_mistakes_fail_a_pin(mutant):
    fn = lambda u, k, D, pts, q, v: short_numpy(u, k, D, pts, q, v, mutant=mutant)
    assert any(not pin(fn) for pin in PINS), mutant


def test_short_oracle_rejects_bad_points():
    u, q, v, k, D = _draw(1, 1, 8, 3, 0)
    with pytest.raises(ValueError):
        oracle.conv1d_short_points(u, k, D, [(0, 0, 8)])

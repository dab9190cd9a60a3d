"""Pins for the 3D oracle (oracle.conv3d_points), CPU only.

The 3D operation is the 2D one a dimension up: a linear convolution with a centred full-size
kernel, cropped to the input window, plus D u ("Native Multi-Dimensional Subquadratic
Operators..." abstract).  Pinned by: a delta kernel at the centre gives (1 + D) u; a shifted
delta gives a shifted copy; the full linear convolution via scipy.signal.convolve
(n-dimensional), cropped; a separable kernel a x b x c reduces to three centred 1D convolutions;
exact integers.  Planted mistakes (an off-centre crop, a flipped kernel axis, a circular wrap, a
dropped skip) each fail a pin.
"""
import numpy as np
import pytest

import oracle


def _draw(B, C, S, seed, integer=False):
    rng = np.random.default_rng(seed)
    if integer:
        f = lambda *s: rng.integers(-3, 4, s).astype(np.float32)
    else:
        f = lambda *s: rng.standard_normal(s).astype(np.float32)
    return f(B, C, S, S, S), f(C, S, S, S), f(C)


def all_pts(B, C, S):
    g = np.stack(np.meshgrid(np.arange(B), np.arange(C), np.arange(S), np.arange(S), np.arange(S),
                             indexing="ij"), -1)
    return g.reshape(-1, 5)


def full_numpy(u, k, D, mutant=None):
    """The definition with explicit index arithmetic (numpy), optionally with a planted mistake."""
    u, k, D = (np.asarray(a, np.float64) for a in (u, k, D))
    B, C, S = u.shape[:3]
    half = S // 2
    if mutant == "flip":
        k = k[:, ::-1]
    y = np.zeros_like(u)
    for a in range(S):
        for e in range(S):
            for f in range(S):
                di, dj, dl = half - a, half - e, half - f
                if mutant == "offcentre":
                    di += 1
                src = u
                if mutant == "circular":
                    y += k[None, :, a, e, f, None, None, None] * np.roll(src, (-di, -dj, -dl), axis=(2, 3, 4))
                    continue
                # y[i] += k[a] u[i + di] where 0 <= i + di < S
                i0, i1 = max(0, -di), min(S, S - di)
                j0, j1 = max(0, -dj), min(S, S - dj)
                l0, l1 = max(0, -dl), min(S, S - dl)
                if i0 < i1 and j0 < j1 and l0 < l1:
                    y[:, :, i0:i1, j0:j1, l0:l1] += k[None, :, a, e, f, None, None, None] * \
                        src[:, :, i0 + di:i1 + di, j0 + dj:j1 + dj, l0 + dl:l1 + dl]
    if mutant != "no_skip":
        y += D[None, :, None, None, None] * u
    return y


def pin_delta_centre(fn):
    u, _, D = _draw(1, 2, 8, 1)
    k = np.zeros((2, 8, 8, 8), np.float32)
    k[:, 4, 4, 4] = 1
    want = (1 + D.astype(np.float64)[None, :, None, None, None]) * u.astype(np.float64)
    return np.allclose(fn(u, k, D), want, rtol=1e-12, atol=1e-12)


def pin_shifted_delta(fn):
    u, _, D = _draw(1, 1, 8, 2)
    D = np.zeros(1, np.float32)
    k = np.zeros((1, 8, 8, 8), np.float32)
    k[0, 5, 4, 2] = 1                      # offset (+1, 0, -2): y[i,j,l] = u[i-1, j, l+2]
    want = np.zeros_like(u, dtype=np.float64)
    want[0, 0, 1:, :, :6] = u[0, 0, :-1, :, 2:]
    return np.allclose(fn(u, k, D), want, rtol=0, atol=0)


def pin_scipy(fn):
    sig = pytest.importorskip("scipy.signal")
    u, k, D = _draw(1, 2, 6, 3)
    S, half = 6, 3
    ref = np.stack([sig.convolve(u[0, c].astype(np.float64), k[c].astype(np.float64), mode="full")
                    [half:half + S, half:half + S, half:half + S] for c in range(2)])[None]
    ref += D.astype(np.float64)[None, :, None, None, None] * u.astype(np.float64)
    return np.allclose(fn(u, k, D), ref, rtol=1e-10, atol=1e-10)


def pin_separable(fn):
    """k = a (x) b (x) c: three centred 1D convolutions, one per axis."""
    rng = np.random.default_rng(4)
    S, half = 8, 4
    u = rng.standard_normal((1, 1, S, S, S)).astype(np.float32)
    # dyadic factors (k/8): the float32 kernel a (x) b (x) c is then exact
    a, b, c = (rng.integers(-16, 17, S).astype(np.float32) / 8 for _ in range(3))
    k = (a[:, None, None] * b[None, :, None] * c[None, None, :])[None]
    D = np.zeros(1, np.float32)

    def conv1(x, w, axis):
        x = np.moveaxis(x, axis, -1)
        out = np.zeros_like(x)
        for t in range(S):
            for s_ in range(S):
                tap = t + half - s_
                if 0 <= tap < S:
                    out[..., t] += w[tap] * x[..., s_]
        return np.moveaxis(out, -1, axis)
    want = conv1(conv1(conv1(u[0, 0].astype(np.float64), a, 0), b, 1), c, 2)[None, None]
    return np.allclose(fn(u, k, D), want, rtol=1e-10, atol=1e-10)


def pin_integer(fn):
    u, k, D = _draw(1, 1, 4, 5, integer=True)
    S, half = 4, 2
    want = np.zeros((S, S, S))
    for i in range(S):
        for j in range(S):
            for l in range(S):
                acc = int(D[0]) * int(u[0, 0, i, j, l])
                for a in range(S):
                    for e in range(S):
                        for f in range(S):
                            ii, jj, ll = i + half - a, j + half - e, l + half - f
                            if 0 <= ii < S and 0 <= jj < S and 0 <= ll < S:
                                acc += int(k[0, a, e, f]) * int(u[0, 0, ii, jj, ll])
                want[i, j, l] = acc
    return np.array_equal(fn(u, k, D)[0, 0], want)


PINS = [pin_delta_centre, pin_shifted_delta, pin_scipy, pin_separable, pin_integer]


def oracle_fn(u, k, D):
    B, C, S = u.shape[:3]
    return oracle.conv3d_points(u, k, D, all_pts(B, C, S)).reshape(u.shape)


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle3d_passes_pins(pin):
    assert pin(oracle_fn)


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_numpy_definition_passes_pins(pin):
    assert pin(lambda u, k, D: full_numpy(u, k, D))


@pytest.mark.parametrize("mutant", ["offcentre", "flip", "circular", "no_skip"])
def test_planted_3d_mistakes_fail_a_pin(mutant):
    assert any(not pin(lambda u, k, D: full_numpy(u, k, D, mutant=mutant)) for pin in PINS), mutant


def test_oracle3d_rejects_bad_points():
    u, k, D = _draw(1, 1, 4, 6)
    with pytest.raises(ValueError):
        oracle.conv3d_points(u, k, D, [(0, 0, 0, 0, 4)])

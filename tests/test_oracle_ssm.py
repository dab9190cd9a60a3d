"""Pins for the state-space filter oracle (oracle.ssm_kernel, oracle.ssm_rows), CPU only.

A diagonal state-space model generates the filter k[t] = Re sum_n W_n lam_n^t ("FlashConv" page,
Mechanism: chunked execution passes the state-space boundary state).  Two independent
definitions are tied together: the state recurrence (ssm_rows) and the causal convolution with
the generated filter (conv1d_circ_rows with the zero-padded k).  Further pins: a real single mode
on a constant input gives the geometric series in closed form; a single complex mode gives
r^t (a cos t theta - b sin t theta).  Planted mistakes (reading the state before adding x[t], a
conjugated mode, a dropped skip) each fail a pin.
"""
import numpy as np
import pytest

import oracle


def _modes(H, NS, seed):
    rng = np.random.default_rng(seed)
    r = np.exp(-rng.uniform(1e-3, 0.2, (H, NS)))
    th = rng.uniform(0, np.pi, (H, NS))
    lam = r * np.exp(1j * th)
    W = (rng.standard_normal((H, NS)) + 1j * rng.standard_normal((H, NS))) / np.sqrt(NS)
    return lam, W


def _draw(B, H, N, seed):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    return f(B, H, N), f(B, H, N), f(B, H, N), f(H)


def rows_of(B, H):
    return [(b, h) for b in range(B) for h in range(H)]


def ssm_numpy(u, lam, W, D, q=None, v=None, mutant=None):
    """The recurrence in numpy (vectorized over modes), optionally wrong."""
    u = np.asarray(u, np.float64)
    B, H, N = u.shape
    x = u * (np.asarray(q, np.float64) if q is not None else 1.0)
    lam = np.asarray(lam, np.complex128)
    if mutant == "conj":
        lam = np.conj(lam)
    y = np.zeros((B, H, N))
    for b in range(B):
        s = np.zeros(lam.shape, np.complex128)
        for t in range(N):
            if mutant == "late":
                y[b, :, t] = (W * s).sum(1).real
                s = lam * s + x[b, :, t][:, None]
            else:
                s = lam * s + x[b, :, t][:, None]
                y[b, :, t] = (W * s).sum(1).real
    if mutant != "no_skip":
        y += np.asarray(D, np.float64)[None, :, None] * x
    if v is not None:
        y *= np.asarray(v, np.float64)
    return y


def pin_recurrence_is_convolution(fn):
    B, H, N, NS = 2, 2, 300, 5
    u, q, v, D = _draw(B, H, N, 1)
    lam, W = _modes(H, NS, 2)
    M = oracle.transform_length(N)
    k = np.zeros((H, M))
    k[:, :N] = oracle.ssm_kernel(lam, W, N)
    ref = oracle.conv1d_circ_rows(u, k, D, rows_of(B, H), q=q, v=v).reshape(B, H, N)
    return np.allclose(fn(u, lam, W, D, q, v), ref, rtol=1e-9, atol=1e-9)


def pin_geometric_series(fn):
    N, a = 200, 0.97
    u = np.ones((1, 1, N), np.float32)
    lam, W = np.asarray([[a + 0j]]), np.asarray([[1 + 0j]])
    D = np.zeros(1, np.float32)
    t = np.arange(N)
    want = (1 - a ** (t + 1)) / (1 - a)
    return np.allclose(fn(u, lam, W, D, None, None)[0, 0], want, rtol=1e-10, atol=1e-10)


def pin_single_complex_mode(fn):
    """A delta input returns the filter: r^t (a cos t th - b sin t th) for W = a + i b."""
    N, r, th, a, b = 150, 0.99, 0.3, 0.7, -0.4
    u = np.zeros((1, 1, N), np.float32)
    u[0, 0, 0] = 1
    lam, W = np.asarray([[r * np.exp(1j * th)]]), np.asarray([[a + 1j * b]])
    D = np.asarray([0.25], np.float32)
    t = np.arange(N)
    want = r ** t * (a * np.cos(t * th) - b * np.sin(t * th))
    want[0] += 0.25
    return np.allclose(fn(u, lam, W, D, None, None)[0, 0], want, rtol=1e-10, atol=1e-10)


PINS = [pin_recurrence_is_convolution, pin_geometric_series, pin_single_complex_mode]


def oracle_fn(u, lam, W, D, q, v):
    B, H, N = u.shape
    return oracle.ssm_rows(u, lam, W, D, rows_of(B, H), q=q, v=v).reshape(B, H, N)


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_ssm_oracle_passes_pins(pin):
    assert pin(oracle_fn)


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_numpy_recurrence_passes_pins(pin):
    assert pin(lambda *a: ssm_numpy(*a))


@pytest.mark.parametrize("mutant", ["late", "conj", "no_skip"])
def test_planted_recurrence_mistakes_fail_a_pin(mutant):
    assert any(not pin(lambda *a: ssm_numpy(*a, mutant=mutant)) for pin in PINS), mutant


def test_ssm_kernel_matches_powers():
    lam, W = _modes(3, 4, 9)
    k = oracle.ssm_kernel(lam, W, 64)
    t = np.arange(64)
    want = (W[:, :, None] * lam[:, :, None] ** t[None, None, :]).sum(1).real
    assert np.allclose(k, want, rtol=1e-12, atol=1e-12)

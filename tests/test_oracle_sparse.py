"""Pins for the frequency-sparse oracle (oracle.sparse_filter + oracle.conv1d_circ_rows), CPU only.

A frequency-sparse convolution keeps the filter spectrum only on some blocks of the
decomposition M = 256 R: the residue classes f mod R ("FlashFFTConv" abstract: frequency-sparse
convolutions skip blocks of the matrix decomposition).  Pinned by:
  * all blocks kept: the causal oracle (the full spectrum changes nothing, and M >= 2N keeps the
    circular sum free of wrap-around);
  * only block 0 kept: the closed form kS[m] = (1/R) sum_r k[(m mod M/R) + r M/R] (keeping every
    R-th frequency periodizes the filter with period M/R);
  * complementary block sets add up to the full convolution (plus one extra D x);
  * a set not closed under r -> R - r is rejected.
Planted mistakes (a band mask f < cutoff instead of residues, a mirrored symmetry rule, a
circular shift of the filter) each fail a pin.
"""
import numpy as np
import pytest

import oracle


def _draw(B, H, N, seed):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    return f(B, H, N), f(B, H, N), f(B, H, N), f(H, N), f(H)


def rows_of(B, H):
    return [(b, h) for b in range(B) for h in range(H)]


def sparse_filter_numpy(k, keep, M, mutant=None):
    """The masking step written with an explicit DFT matrix (no FFT), optionally wrong."""
    H, N = k.shape
    R = M // 256
    n = np.arange(M)
    W = np.exp(-2j * np.pi * np.outer(n, n) / M)
    pad = np.zeros((H, M))
    pad[:, :N] = k
    K = pad @ W.T
    if mutant == "band":
        mask = np.isin(n // (M // R), keep)
    else:
        mask = np.isin(n % R, keep)
    kS = ((K * mask[None, :]) @ np.conj(W).T / M).real
    if mutant == "shift":
        kS = np.roll(kS, 1, axis=1)
    return kS


def pin_all_blocks_is_causal(sf):
    u, q, v, k, D = _draw(2, 2, 40, 1)
    M = oracle.transform_length(40)
    kS = sf(k, range(M // 256), M)
    got = oracle.conv1d_circ_rows(u, kS, D, rows_of(2, 2), q=q, v=v)
    ref = oracle.conv1d_rows(u, k, D, rows_of(2, 2), q=q, v=v)
    return np.allclose(got, ref, rtol=1e-10, atol=1e-10)


def pin_block0_periodizes(sf):
    _, _, _, k, _ = _draw(1, 2, 300, 2)       # N = 300 -> M = 1024, R = 4, period 256
    M = oracle.transform_length(300)
    R, P = M // 256, 256
    pad = np.zeros((2, M))
    pad[:, :300] = k.astype(np.float64)
    want = pad.reshape(2, R, P).sum(axis=1)[:, np.arange(M) % P] / R
    return np.allclose(sf(k, [0], M), want, rtol=1e-10, atol=1e-12)


def pin_complement_adds(sf):
    u, q, v, k, D = _draw(1, 2, 1000, 3)      # M = 2048, R = 8
    M = oracle.transform_length(1000)
    R = M // 256
    S = [0, 1, 7, 3, 5]                       # closed under r -> R - r
    Sc = [r for r in range(R) if r not in S]
    rows = rows_of(1, 2)
    yS = oracle.conv1d_circ_rows(u, sf(k, S, M), D, rows, q=q, v=v)
    yC = oracle.conv1d_circ_rows(u, sf(k, Sc, M), D, rows, q=q, v=v)
    yA = oracle.conv1d_rows(u, k, D, rows, q=q, v=v)
    x = (u.astype(np.float64) * q)[0]
    dx = D.astype(np.float64)[:, None] * x * v[0]
    return np.allclose(yS + yC - dx, yA, rtol=1e-9, atol=1e-9)


PINS = [pin_all_blocks_is_causal, pin_block0_periodizes, pin_complement_adds]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_sparse_oracle_passes_pins(pin):
    assert pin(lambda k, keep, M: oracle.sparse_filter(k, keep, M))


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_explicit_dft_masking_passes_pins(pin):
    assert pin(lambda k, keep, M: sparse_filter_numpy(k.astype(np.float64), list(keep), M))


@pytest.mark.parametrize("mutant", ["band", "shift"])
def test_planted_masking_mistakes_fail_a_pin(mutant):
    fn = lambda k, keep, M: sparse_filter_numpy(k.astype(np.float64), list(keep), M, mutant=mutant)
    assert any(not pin(fn) for pin in PINS), mutant


def test_mirrored_symmetry_rule_is_rejected():
    _, _, _, k, _ = _draw(1, 1, 64, 4)        # M = 512, R = 2: any set is closed
    k2 = np.zeros((1, 1000), np.float32)      # M = 2048, R = 8
    with pytest.raises(ValueError):
        oracle.sparse_filter(k2, [1, 6], 2048)  # the mirror of 1 is 7, not 6 (R - 1 - r)
    with pytest.raises(ValueError):
        oracle.sparse_filter(k2, [8], 2048)
    assert oracle.sparse_filter(k, [0, 1], 512).shape == (1, 512)


def test_circ_rows_rejects_short_transform():
    u, q, v, k, D = _draw(1, 1, 64, 5)
    with pytest.raises(ValueError):
        oracle.conv1d_circ_rows(u, np.zeros((1, 100)), D, [(0, 0)])

"""Pins for the learned-Butterfly oracle (CPU only).

The page ("Simple Hardware-Efficient Long Convolutions for Sequence Modeling", abstract) says
only that the Butterfly decomposition's coefficients are learned, so the pins are structural:
  * with the DFT's own blocks the map is the DFT (numpy FFT) and the convolution is the causal
    sum of the plain oracle (a closed-form reduction);
  * for random blocks the staged contractions equal the dense matrices written entry by entry
    from the path formula T[f, n] = A3 w256 A2 A1 (and S for the inverse) -- an independent
    construction, not a re-run of the staged code;
  * the flat ABI order unpacks into the named blocks;
  * planted mistakes (a transposed block, the twiddle conjugated, a swapped digit order)
    each fail one of these pins.
"""
import numpy as np
import pytest

import oracle
from oracle import butterfly as bf

RNG = np.random.default_rng(2024)


def rand_blocks(M, scale=1.0, rng=RNG):
    R = M // 256
    def c(*shape):
        return scale * (rng.standard_normal(shape) + 1j * rng.standard_normal(shape))
    return {"A1": c(R, R), "A2": c(R, 16, 16), "A3": c(R, 16, 16),
            "B1": c(R, 16, 16), "B2": c(R, 16, 16), "B3": c(R, R)}


@pytest.mark.parametrize("M", [512, 1024, 8192])
def test_dft_blocks_give_the_dft(M):
    bl = bf.dft_blocks(M)
    x = RNG.standard_normal((3, M)) + 1j * RNG.standard_normal((3, M))
    np.testing.assert_allclose(bf.forward(x, bl), np.fft.fft(x, axis=-1), rtol=0, atol=1e-9 * M)
    np.testing.assert_allclose(bf.inverse(x, bl), M * np.fft.ifft(x, axis=-1), rtol=0, atol=1e-9 * M)


@pytest.mark.parametrize("N", [8, 200, 256, 1000, 4096])
def test_dft_blocks_give_the_causal_convolution(N):
    B, H = 2, 3
    u = RNG.standard_normal((B, H, N)).astype(np.float32)
    q = RNG.standard_normal((B, H, N)).astype(np.float32)
    v = RNG.standard_normal((B, H, N)).astype(np.float32)
    k = (RNG.standard_normal((H, N)) * np.exp(-np.arange(N) / 50.0)).astype(np.float32)
    D = RNG.standard_normal(H).astype(np.float32)
    got = bf.butterfly_conv(u, k, D, bf.dft_blocks(oracle.transform_length(N)), q=q, v=v)
    rows = [(b, h) for b in range(B) for h in range(H)]
    ref = oracle.conv1d_rows(u, k, D, rows, q=q, v=v).reshape(B, H, N)
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())


@pytest.mark.parametrize("M", [512, 1024])
def test_staged_equals_dense_entrywise(M):
    bl = rand_blocks(M)
    T, S = bf.dense(bl, M)
    x = RNG.standard_normal((2, M)) + 1j * RNG.standard_normal((2, M))
    np.testing.assert_allclose(bf.forward(x, bl), x @ T.T, rtol=1e-10, atol=1e-9 * np.abs(x @ T.T).max())
    np.testing.assert_allclose(bf.inverse(x, bl), x @ S.T, rtol=1e-10, atol=1e-9 * np.abs(x @ S.T).max())


def test_dense_of_dft_blocks_is_the_dft_matrix():
    M = 512
    T, S = bf.dense(bf.dft_blocks(M), M)
    F = np.exp(-2j * np.pi * (np.outer(np.arange(M), np.arange(M)) % M) / M)
    np.testing.assert_allclose(T, F, atol=1e-12)
    np.testing.assert_allclose(S, np.conj(F), atol=1e-12)


def test_convolution_with_random_blocks_matches_dense():
    """y = Re(S diag(K) T x)[:N] + D x with T, S dense: the convolution uses the staged maps
    exactly as defined."""
    N, M = 200, 512
    bl = rand_blocks(M, 0.1)
    u = RNG.standard_normal((1, 2, N)).astype(np.float32)
    k = RNG.standard_normal((2, N)).astype(np.float32)
    D = RNG.standard_normal(2).astype(np.float32)
    got = bf.butterfly_conv(u, k, D, bl)
    T, S = bf.dense(bl, M)
    for h in range(2):
        x = np.zeros(M); x[:N] = u[0, h]
        kp = np.zeros(M); kp[:N] = k[h]
        K = T @ kp / M
        y = (S @ (K * (T @ x))).real[:N] + float(D[h]) * u[0, h].astype(np.float64)
        np.testing.assert_allclose(got[0, h], y, rtol=1e-9, atol=1e-9 * np.abs(y).max())


def test_flat_order_unpacks_into_named_blocks():
    M = 1024
    R = M // 256
    bl = rand_blocks(M)
    flat = np.concatenate([bl[n].ravel() for n in ("A1", "A2", "A3", "B1", "B2", "B3")])
    assert flat.size == 2 * R * R + 4 * 256 * R
    back = bf.unpack_blocks(flat, M)
    for n in bl:
        np.testing.assert_array_equal(back[n], bl[n])


# ---- planted mistakes: each must break a pin -------------------------------------------------

def _forward_mutant(kind):
    def fwd(x, bl):
        M = x.shape[-1]
        R = M // 256
        xs = x.reshape(x.shape[:-1] + (R, 16, 16))
        A2 = np.swapaxes(bl["A2"], 1, 2) if kind == "A2T" else bl["A2"]
        a = np.einsum("kn,...nbc->...kbc", bl["A1"], xs)
        b = np.einsum("kpn,...knc->...kpc", A2, a)
        tw = bf._w256()
        c = b * (np.conj(tw) if kind == "tw" else tw)  # "tw": the twiddle's sign flipped
        X = np.einsum("kqc,...kpc->...kpq", bl["A3"], c)
        if kind == "order":
            return X.reshape(x.shape[:-1] + (M,))  # k1 slowest instead of k3
        return np.moveaxis(X, (-3, -2, -1), (-1, -2, -3)).reshape(x.shape[:-1] + (M,))
    return fwd


@pytest.mark.parametrize("kind", ["A2T", "tw", "order"])
def test_planted_mistakes_fail_a_pin(kind):
    M = 512
    fwd = _forward_mutant(kind)
    x = RNG.standard_normal(M) + 1j * RNG.standard_normal(M)
    bl_dft, bl_rand = bf.dft_blocks(M), rand_blocks(M)
    T, _ = bf.dense(bl_rand, M)
    ok_dft = np.allclose(fwd(x, bl_dft), np.fft.fft(x), atol=1e-9 * M)
    ok_dense = np.allclose(fwd(x, bl_rand), T @ x, atol=1e-9 * np.abs(T @ x).max())
    assert not (ok_dft and ok_dense)

"""Pins for the float64 CPU oracle (CPU only).

The pages print no worked example or test vector, so every pin here is definitional: special
inputs with closed-form answers, exact integer brute force, algebraic invariants, and
reductions to textbook library routines.  Each pin is written as a function of a convolution
callable so that the same pins can be run against deliberately broken variants (planted
mistakes, on the CPU): every variant must fail at least one pin.

Definition pinned (restated from "FlashFFTConv" abstract -- exact FFT convolution -- and the
Caracal abstract on the "RubiConv" page -- causality by one-sided padding and truncation):
    y[b,h,t] = v * ( sum_{s<=t} k[h,t-s] x[b,h,s] + D[h] x[b,h,t] ),  x = q*u
2D ("Native Multi-Dimensional Subquadratic Operators..." abstract): centred full-size kernel,
linear convolution cropped to the input window.
"""
import numpy as np
import pytest
import scipy.fft
import scipy.signal

import oracle
from fft_long_convolution_amd import workloads as wl

RNG = np.random.default_rng(12345)


# --------------------------------------------------------------------------------------------
# Convolution callables: the oracle and planted-mistake variants (numpy, small sizes only)
# --------------------------------------------------------------------------------------------

def conv_oracle(u, k, D, q=None, v=None):
    """Full rows from the C oracle; u:[B,H,N] float32, k:[H,N], D:[H]."""
    B, H, N = u.shape
    rows = [(b, h) for b in range(B) for h in range(H)]
    return oracle.conv1d_rows(u, k, D, rows, q=q, v=v).reshape(B, H, N)


def _mutant(kind):
    def conv(u, k, D, q=None, v=None):
        B, H, N = u.shape
        x = u.astype(np.float64) * (1.0 if q is None else q.astype(np.float64))
        kk = k.astype(np.float64)
        y = np.zeros((B, H, N))
        for b in range(B):
            for h in range(H):
                for t in range(N):
                    acc = 0.0
                    for s in range(N):
                        lag = t - s
                        if kind == "circular":
                            lag %= N
                        elif kind == "anticausal":
                            lag = s - t
                        elif kind == "lag_off_by_one":
                            lag = t - s - 1
                        if 0 <= lag < N and (kind in ("circular", "anticausal") or s <= t):
                            acc += kk[h, lag] * x[b, h, s]
                    d = 0.0 if kind == "no_skip" else float(D[h])
                    skip = d * (u[b, h, t] if kind == "skip_ungated" else x[b, h, t])
                    val = acc + skip
                    if v is not None and kind != "gate_dropped":
                        val *= float(v[b, h, t])
                    y[b, h, t] = val
        return y
    return conv


MUTANTS = ["circular", "anticausal", "lag_off_by_one", "no_skip", "skip_ungated", "gate_dropped"]


def _f32(a):
    return np.ascontiguousarray(a, np.float32)


# --------------------------------------------------------------------------------------------
# Pins (each returns None on success, raises AssertionError on failure)
# --------------------------------------------------------------------------------------------

def pin_delta_input(conv, N=24):
    """u = e_0, D = 0  =>  y[h,:] = k[h,:] exactly (lag indexing and kernel orientation)."""
    H = 3
    u = np.zeros((1, H, N), np.float32); u[..., 0] = 1
    k = _f32(RNG.standard_normal((H, N)))
    y = conv(u, k, np.zeros(H, np.float32))
    assert np.array_equal(y[0], k.astype(np.float64))


def pin_delta_filter(conv, N=20):
    """k = e_0  =>  y = v * (x + D x) with x = q u (skip term and gating order)."""
    B, H = 2, 3
    u = _f32(RNG.standard_normal((B, H, N)))
    q = _f32(RNG.standard_normal((B, H, N)))
    v = _f32(RNG.standard_normal((B, H, N)))
    k = np.zeros((H, N), np.float32); k[:, 0] = 1
    D = _f32(RNG.standard_normal(H))
    y = conv(u, k, D, q=q, v=v)
    x = u.astype(np.float64) * q.astype(np.float64)
    ref = (x + D.astype(np.float64)[None, :, None] * x) * v.astype(np.float64)
    np.testing.assert_allclose(y, ref, rtol=1e-15, atol=0)
    y2 = conv(u, k, D)
    ref2 = u.astype(np.float64) * (1 + D.astype(np.float64))[None, :, None]
    np.testing.assert_allclose(y2, ref2, rtol=1e-15, atol=0)


def pin_causal_discriminator(conv, N=16):
    """u = k = e_{N-1}, D = 0  =>  y = 0 (a circular length-N convolution would put a 1 at
    t = N-2); u = e_{N-1}, k = e_0  =>  y = e_{N-1}."""
    u = np.zeros((1, 1, N), np.float32); u[..., N - 1] = 1
    k = np.zeros((1, N), np.float32); k[0, N - 1] = 1
    y = conv(u, k, np.zeros(1, np.float32))
    assert np.array_equal(y, np.zeros_like(y))
    k2 = np.zeros((1, N), np.float32); k2[0, 0] = 1
    y2 = conv(u, k2, np.zeros(1, np.float32))
    assert np.array_equal(y2[0, 0], u[0, 0].astype(np.float64))
    # future input must not leak into the past
    u3 = np.zeros((1, 1, N), np.float32); u3[..., 5] = 1
    k3 = _f32(RNG.standard_normal((1, N)))
    y3 = conv(u3, k3, np.zeros(1, np.float32))
    assert np.all(y3[..., :5] == 0)


def pin_brute_force_int(conv, N=40):
    """Integer-valued u, k, D in [-8, 8]: bit-exact against Python ints and a Toeplitz matvec."""
    B, H = 2, 3
    u = RNG.integers(-8, 9, (B, H, N)).astype(np.float32)
    k = RNG.integers(-8, 9, (H, N)).astype(np.float32)
    D = RNG.integers(-8, 9, H).astype(np.float32)
    y = conv(u, k, D)
    for b in range(B):
        for h in range(H):
            exact = oracle.conv1d_python_int(u[b, h].astype(int), k[h].astype(int), int(D[h]))
            assert np.array_equal(y[b, h], np.asarray(exact, np.float64))
            assert np.array_equal(y[b, h], oracle.conv1d_toeplitz(
                u[b, h].astype(np.float64), k[h].astype(np.float64), float(D[h])))


def pin_closed_form(conv, N=48):
    """k[t] = 2^-t, u = 1  =>  y[t] = 2 - 2^-t + D (exact in binary floating point)."""
    u = np.ones((1, 1, N), np.float32)
    k = (0.5 ** np.arange(N)).astype(np.float32)[None]
    D = np.array([0.25], np.float32)
    y = conv(u, k, D)[0, 0]
    t = np.arange(N, dtype=np.float64)
    assert np.array_equal(y, 2.0 - 2.0 ** (-t) + 0.25)


def pin_shift_equivariance(conv, N=32, s=7):
    """Delaying u, q, v by s (zero fill) delays y by s and leaves zeros before s."""
    B, H = 1, 2
    u = _f32(RNG.standard_normal((B, H, N)))
    q = _f32(RNG.standard_normal((B, H, N)))
    v = _f32(RNG.standard_normal((B, H, N)))
    k = _f32(RNG.standard_normal((H, N)))
    D = _f32(RNG.standard_normal(H))
    sh = lambda a: np.concatenate([np.zeros_like(a[..., :s]), a[..., :-s]], axis=-1)
    y = conv(u, k, D, q=q, v=v)
    y2 = conv(sh(u), k, D, q=sh(q), v=sh(v))
    assert np.all(y2[..., :s] == 0)
    assert np.array_equal(y2[..., s:], y[..., :-s])


def pin_linearity(conv, N=32):
    """y is linear in u (and in k): exact-integer combinations, float64 tolerance 1e-12."""
    H = 2
    u1 = RNG.integers(-8, 9, (1, H, N)).astype(np.float32)
    u2 = RNG.integers(-8, 9, (1, H, N)).astype(np.float32)
    k = _f32(RNG.standard_normal((H, N)))
    D = _f32(RNG.standard_normal(H))
    lhs = conv(3 * u1 - 2 * u2, k, D)
    rhs = 3 * conv(u1, k, D) - 2 * conv(u2, k, D)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    # linearity in k: dyadic filters so that k1 + k2 is exact in float32
    Z = np.zeros(H, np.float32)
    k1 = (RNG.integers(-64, 65, (H, N)) / 16).astype(np.float32)
    k2 = (RNG.integers(-64, 65, (H, N)) / 16).astype(np.float32)
    u3 = _f32(RNG.standard_normal((1, H, N)))
    lhs = conv(u3, k1 + k2, Z)
    rhs = conv(u3, k1, Z) + conv(u3, k2, Z)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def pin_library(conv, N=64):
    """numpy.convolve(x, k)[:N] and a scipy rfft/irfft product at length 2N agree (1e-12)."""
    B, H = 2, 3
    u = _f32(RNG.standard_normal((B, H, N)))
    q = _f32(RNG.standard_normal((B, H, N)))
    v = _f32(RNG.standard_normal((B, H, N)))
    k = _f32(RNG.standard_normal((H, N)))
    D = _f32(RNG.standard_normal(H))
    y = conv(u, k, D, q=q, v=v)
    x = u.astype(np.float64) * q
    for b in range(B):
        for h in range(H):
            c = np.convolve(x[b, h], k[h].astype(np.float64))[:N]
            ref = (c + float(D[h]) * x[b, h]) * v[b, h]
            np.testing.assert_allclose(y[b, h], ref, rtol=1e-12, atol=1e-12)
            f = scipy.fft.irfft(scipy.fft.rfft(x[b, h], 2 * N) *
                                scipy.fft.rfft(k[h].astype(np.float64), 2 * N), 2 * N)[:N]
            ref = (f + float(D[h]) * x[b, h]) * v[b, h]
            np.testing.assert_allclose(y[b, h], ref, rtol=1e-11, atol=1e-11)


PINS = [pin_delta_input, pin_delta_filter, pin_causal_discriminator, pin_brute_force_int,
        pin_closed_form, pin_shift_equivariance, pin_linearity, pin_library]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pins(pin):
    pin(conv_oracle)


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistakes_are_caught(kind):
    conv = _mutant(kind)
    failed = []
    for pin in PINS:
        try:
            pin(conv)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake '{kind}'"


def test_correct_numpy_variant_passes_pins():
    """The mutant harness itself, with no mistake planted, passes every pin."""
    for pin in PINS:
        pin(_mutant("none"))


# --------------------------------------------------------------------------------------------
# Sampled evaluator, widening and input-dtype handling
# --------------------------------------------------------------------------------------------

def test_points_match_rows_bitwise():
    """Sampled positions equal the same positions of full rows, bit for bit."""
    spec = wl.spec_1d(3, 5, 1000, "bf16", gated=True, seed=3)
    d = wl.make(spec)
    full = oracle.conv1d_rows(d["u"], d["k"], d["D"], [(b, h) for b in range(3) for h in range(5)],
                              q=d["q"], v=d["v"], dt=oracle.DT_BF16).reshape(3, 5, 1000)
    pts = wl.sample_points_1d(3, 5, 1000, n_uniform=300, n_struct=64, seed=9)
    got = oracle.conv1d_points(d["u"], d["k"], d["D"], pts, q=d["q"], v=d["v"], dt=oracle.DT_BF16)
    assert np.array_equal(got, full[pts[:, 0], pts[:, 1], pts[:, 2]])


def test_widen_f16_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    h = bits.view(np.float16)
    finite = np.isfinite(h)
    got = oracle.widen(h[finite])
    assert np.array_equal(got, h[finite].astype(np.float64))
    assert np.all(np.isinf(oracle.widen(h[np.isinf(h)])))


def test_widen_bf16_matches_bit_layout():
    bits = RNG.integers(0, 65536, 100000).astype(np.uint16)
    f = wl.bf16_bits_to_f32(bits)
    ok = np.isfinite(f)
    got = oracle.widen(bits[ok], oracle.DT_BF16)
    assert np.array_equal(got, f[ok].astype(np.float64))


def test_dtype_inputs_are_widened_exactly():
    """The oracle on bf16/fp16 inputs equals the oracle on their exact float32 values."""
    for dt in ("bf16", "f16"):
        spec = wl.spec_1d(2, 3, 256, dt, gated=True, seed=11)
        d = wl.make(spec)
        code = oracle.DT_BF16 if dt == "bf16" else oracle.DT_F16
        rows = [(b, h) for b in range(2) for h in range(3)]
        y = oracle.conv1d_rows(d["u"], d["k"], d["D"], rows, q=d["q"], v=d["v"], dt=code)
        f32 = lambda a: wl.storage_to_f64(a, dt).astype(np.float32)
        y32 = oracle.conv1d_rows(f32(d["u"]), f32(d["k"]), f32(d["D"]), rows,
                                 q=f32(d["q"]), v=f32(d["v"]))
        assert np.array_equal(y, y32)


def test_rejects_bad_arguments():
    u = np.zeros((1, 2, 8), np.float32)
    k = np.zeros((2, 8), np.float32)
    D = np.zeros(2, np.float32)
    with pytest.raises(ValueError):
        oracle.conv1d_rows(u, k, D, [(0, 2)])
    with pytest.raises(ValueError):
        oracle.conv1d_points(u, k, D, [(0, 0, 8)])


# --------------------------------------------------------------------------------------------
# 2D pins
# --------------------------------------------------------------------------------------------

def _img_all_points(B, C, Hs, Ws):
    g = np.stack(np.meshgrid(np.arange(B), np.arange(C), np.arange(Hs), np.arange(Ws),
                             indexing="ij"), -1)
    return g.reshape(-1, 4)


def _conv2d_direct_full(u, k, D):
    B, C, Hs, Ws = u.shape
    return oracle.conv2d_points(u, k, D, _img_all_points(B, C, Hs, Ws)).reshape(B, C, Hs, Ws)


# square, rectangular, odd sides (centre tap at the rounded-down half)
SHAPES_2D = [(16, 16), (8, 24), (9, 16), (12, 7), (1, 8)]


@pytest.mark.parametrize("Hs,Ws", SHAPES_2D)
@pytest.mark.parametrize("which", ["direct", "dft"])
def test_2d_delta_at_centre_is_identity_plus_skip(which, Hs, Ws):
    B, C = 2, 3
    u = _f32(RNG.standard_normal((B, C, Hs, Ws)))
    k = np.zeros((C, Hs, Ws), np.float32); k[:, Hs // 2, Ws // 2] = 1
    D = _f32(RNG.standard_normal(C))
    y = (_conv2d_direct_full(u, k, D) if which == "direct" else
         oracle.conv2d_dft(u, k, D, [(b, c) for b in range(B) for c in range(C)]).reshape(B, C, Hs, Ws))
    ref = u.astype(np.float64) * (1 + D.astype(np.float64))[None, :, None, None]
    tol = 0 if which == "direct" else 1e-12
    np.testing.assert_allclose(y, ref, rtol=tol, atol=tol)


@pytest.mark.parametrize("Hs,Ws", SHAPES_2D)
@pytest.mark.parametrize("which", ["direct", "dft"])
def test_2d_shifted_delta_is_shifted_copy(which, Hs, Ws):
    dx, dy = min(3, Hs - 1 - Hs // 2), -min(2, Ws // 2)
    u = _f32(RNG.standard_normal((1, 1, Hs, Ws)))
    k = np.zeros((1, Hs, Ws), np.float32); k[0, Hs // 2 + dx, Ws // 2 + dy] = 1
    D = np.zeros(1, np.float32)
    if which == "direct":
        y = _conv2d_direct_full(u, k, D)[0, 0]
    else:
        y = oracle.conv2d_dft(u, k, D, [(0, 0)])[0]
    ref = np.zeros((Hs, Ws))
    for i in range(Hs):
        for j in range(Ws):
            ii, jj = i - dx, j - dy
            if 0 <= ii < Hs and 0 <= jj < Ws:
                ref[i, j] = u[0, 0, ii, jj]
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("Hs,Ws", SHAPES_2D)
def test_2d_matches_scipy_convolve2d_crop(Hs, Ws):
    B, C = 2, 2
    u = _f32(RNG.standard_normal((B, C, Hs, Ws)))
    k = _f32(RNG.standard_normal((C, Hs, Ws)))
    D = _f32(RNG.standard_normal(C))
    yd = _conv2d_direct_full(u, k, D)
    yf = oracle.conv2d_dft(u, k, D, [(b, c) for b in range(B) for c in range(C)]).reshape(B, C, Hs, Ws)
    h, w = Hs // 2, Ws // 2
    for b in range(B):
        for c in range(C):
            full = scipy.signal.convolve2d(u[b, c].astype(np.float64), k[c].astype(np.float64),
                                           mode="full")
            ref = full[h:h + Hs, w:w + Ws] + float(D[c]) * u[b, c].astype(np.float64)
            np.testing.assert_allclose(yd[b, c], ref, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(yf[b, c], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("Hs,Ws", SHAPES_2D)
def test_2d_separable_kernel_reduces_to_1d_centred_convs(Hs, Ws):
    u = _f32(RNG.standard_normal((1, 1, Hs, Ws)))
    f = RNG.integers(-4, 5, Hs).astype(np.float32)
    g = RNG.integers(-4, 5, Ws).astype(np.float32)
    k = np.outer(f, g).astype(np.float32)[None]
    y = _conv2d_direct_full(u, k, np.zeros(1, np.float32))[0, 0]
    # rows with g, then columns with f; each a centred 1D linear conv cropped at the half
    tmp = np.stack([np.convolve(r, g.astype(np.float64))[Ws // 2:Ws // 2 + Ws]
                    for r in u[0, 0].astype(np.float64)])
    ref = np.stack([np.convolve(col, f.astype(np.float64))[Hs // 2:Hs // 2 + Hs]
                    for col in tmp.T]).T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_2d_dft_larger_padding_agrees():
    """Any padding Ph >= 2Hs - 1, Pw >= 2Ws - 1 gives the same linear convolution."""
    u = _f32(RNG.standard_normal((1, 2, 9, 12)))
    k = _f32(RNG.standard_normal((2, 9, 12)))
    D = _f32(RNG.standard_normal(2))
    a = oracle.conv2d_dft(u, k, D, [(0, 0), (0, 1)])
    b = oracle.conv2d_dft(u, k, D, [(0, 0), (0, 1)], P=(17, 30))
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_2d_dft_matches_direct_at_sampled_points_full_size():
    """S = 128 as in the 2D workload: naive DFT vs direct sums at 256 sampled positions."""
    spec = wl.Conv2DSpec("t", 2, 3, 128, "bf16", seed=5)
    d = wl.make(spec)
    pts = wl.sample_points_2d(2, 3, 128, n=256, seed=1)
    yd = oracle.conv2d_points(d["u"], d["k"], d["D"], pts, dt=oracle.DT_BF16)
    imgs = sorted({(int(b), int(c)) for b, c in pts[:, :2]})
    yf = oracle.conv2d_dft(d["u"], d["k"], d["D"], imgs, dt=oracle.DT_BF16)
    idx = {im: n for n, im in enumerate(imgs)}
    got = np.array([yf[idx[(int(b), int(c))], i, j] for b, c, i, j in pts])
    np.testing.assert_allclose(got, yd, rtol=1e-12, atol=1e-10)

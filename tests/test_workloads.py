"""Seeded input generator: determinism, round-to-nearest-even casts, workload recipes (CPU)."""
import numpy as np
import pytest
import torch

from fft_long_convolution_amd import workloads as wl


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(500000).astype(np.float32),
                        (rng.standard_normal(500000) * 1e-3).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 3.0, 65504.0, 1e-30], np.float32)])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_from_f64_single_rounding():
    # a value just above a bf16 tie in float64 that float32 would round onto the tie
    one = 1.0
    tie = one + 2.0 ** -8                   # exactly halfway between 1 and 1 + 2^-7
    x = np.array([tie + 2.0 ** -40, tie, tie - 2.0 ** -40, -tie - 2.0 ** -40])
    got = wl.bf16_bits_to_f32(wl.f64_to_bf16_bits(x)).astype(np.float64)
    assert got[0] == 1 + 2.0 ** -7          # above the tie: round up
    assert got[1] == 1.0                    # tie: to even
    assert got[2] == 1.0
    assert got[3] == -(1 + 2.0 ** -7)
    rng = np.random.default_rng(1)
    y = rng.standard_normal(100000) * 10.0 ** rng.integers(-6, 6, 100000)
    b = wl.bf16_bits_to_f32(wl.f64_to_bf16_bits(y)).astype(np.float64)
    # nearest representable: error at most half an ulp of an 8-bit significand
    m, e = np.frexp(y)
    assert np.all(np.abs(b - y) <= np.ldexp(1.0, e - 9) * (1 + 1e-12))


def test_same_bytes_for_same_seed():
    spec = wl.spec_1d(2, 3, 64, "bf16", gated=True, seed=42)
    a, b = wl.make(spec), wl.make(spec)
    for key in ("u", "q", "v", "k", "D"):
        assert np.array_equal(a[key], b[key])
    c = wl.make(wl.spec_1d(2, 3, 64, "bf16", gated=True, seed=43))
    assert not np.array_equal(a["u"], c["u"])


def test_workload_shapes_and_dtypes():
    d = wl.make("causal_f32_b1_h4_n1024")
    assert d["u"].shape == (1, 4, 1024) and d["u"].dtype == np.float32
    assert d["k"].shape == (4, 1024) and d["D"].shape == (4,)
    assert d["q"] is None and d["v"] is None
    spec = wl.WORKLOADS["hyena_gated_bf16_b16_h768_n4096"]
    assert (spec.B, spec.H, spec.N, spec.dtype, spec.gated) == (16, 768, 4096, "bf16", True)
    assert wl.WORKLOADS["long_f16_b4_h256_n65536"].dtype == "f16"
    assert wl.WORKLOADS["very_long_bf16_b1_h64_n2097152"].N == 2 ** 21
    s2 = wl.WORKLOADS["hyenand_2d_bf16_b8_c256_s128"]
    assert (s2.B, s2.C, s2.S) == (8, 256, 128)


def test_filter_recipe_squash_and_envelope():
    spec = wl.spec_1d(1, 2, 512, "f32", decay=0.01, squash_lam=0.01, seed=5)
    d = wl.make(spec)
    k = d["k"].astype(np.float64)
    # squashed: no value in (0, 0) band is possible beyond float32 rounding; zeros appear
    assert np.mean(k == 0) > 0.01
    # envelope: late taps are tiny
    assert np.max(np.abs(k[:, 400:])) < 0.05
    # redraw by hand from the same seed: draw order u, k_raw, D
    rng = np.random.default_rng(5)
    rng.standard_normal((1, 2, 512), dtype=np.float32)
    kr = rng.standard_normal((2, 512)) * np.exp(-0.01 * np.arange(512))
    kr = np.sign(kr) * np.maximum(np.abs(kr) - 0.01, 0)
    assert np.array_equal(d["k"], kr.astype(np.float32))


def test_sample_points_in_range_and_structured():
    pts = wl.sample_points_1d(4, 256, 65536, seed=2003)
    assert pts.shape == (4096, 3)
    assert pts[:, 0].max() < 4 and pts[:, 1].max() < 256 and pts[:, 2].max() < 65536
    ts = set(pts[:, 2].tolist())
    assert {0, 1, 65534, 65535} <= ts
    assert any(t % 256 == 255 for t in ts) and any(t % 4096 == 0 and t > 0 for t in ts)
    p2 = wl.sample_points_2d(8, 256, 128)
    assert p2.shape == (4096, 4) and p2[:, 2:].max() < 128


def test_short_filter_workload_draws_l_taps():
    spec = wl.spec_partial(2, 3, 256, 24, "bf16", gated=True, seed=3)
    d = wl.make(spec)
    assert d["k"].shape == (3, 24) and d["u"].shape == (2, 3, 256)
    assert spec.taps == 24 and wl.spec_1d(1, 1, 64, "f32").taps == 64
    long = wl.WORKLOADS["partial_bf16_b1_h64_n2097152_l4096"]
    assert (long.N, long.L, long.dtype) == (2 ** 21, 4096, "bf16")


def test_3d_workload_draws():
    spec = wl.spec_3d(3, 2, 16, "f32", seed=5)
    d = wl.make(spec)
    assert d["u"].shape == (3, 2, 16, 16, 16) and d["k"].shape == (2, 16, 16, 16)
    assert d["D"].shape == (2,)
    k = d["k"].astype(np.float64)
    assert np.abs(k[:, 8, 8, 8]).mean() > np.abs(k[:, 0, 0, 0]).mean()   # centred envelope
    pts = wl.sample_points_3d(3, 2, 16)
    assert pts.shape[1] == 5 and pts[:, 2:].max() < 16

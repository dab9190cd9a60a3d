"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random numbers and rounds them to the storage dtype; it holds none of
the convolution's arithmetic.  Both the HIP path (through the tests and the bench) and the CPU
oracle take their inputs from here.

Filters follow "Simple Hardware-Efficient Long Convolutions for Sequence Modeling" (abstract):
long per-channel kernels kept smooth by an exponential envelope and, where a workload asks for
it, the squashing step k <- sign(k) * max(|k| - lambda, 0).  The 2D workload follows "Native
Multi-Dimensional Subquadratic Operators via Input Dependent Long Convolutions" (abstract):
global, full-size kernels on a native image grid.

Storage dtypes: ``"f32"`` -> numpy float32, ``"f16"`` -> numpy float16, ``"bf16"`` -> numpy
uint16 holding bfloat16 bit patterns.  Every cast rounds to nearest, ties to even.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

DTYPES = ("f32", "f16", "bf16")


# --------------------------------------------------------------------------------------------
# Round-to-nearest-even casts
# --------------------------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bits with a single rounding to 8 significant bits (ties to even).

    The value is first rounded to 8 significant bits in float64 (exact: frexp, rint, ldexp),
    which is then exactly representable in float32 and therefore in bfloat16.  Values below
    the float32 normal range take float32's rounding once more; the workloads here never
    depend on such tiny values.
    """
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                          # x = m * 2^e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(m * 256.0), e - 8)     # 8 significant bits, RNE
    return f32_to_bf16_bits(r.astype(np.float32))


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32/float64 values to the storage dtype (RNE)."""
    x = np.asarray(x)
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16)          # numpy rounds float64/float32 -> half RNE
    if dtype == "bf16":
        return f64_to_bf16_bits(x) if x.dtype == np.float64 else f32_to_bf16_bits(x)
    raise ValueError(dtype)


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a).astype(np.float64)


# --------------------------------------------------------------------------------------------
# Filters
# --------------------------------------------------------------------------------------------

def squash(k: np.ndarray, lam: float) -> np.ndarray:
    """k <- sign(k) * max(|k| - lam, 0) (the smoothing intervention of the long-conv paper)."""
    return np.sign(k) * np.maximum(np.abs(k) - lam, 0.0)


# --------------------------------------------------------------------------------------------
# Workload descriptions
# --------------------------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Conv1DSpec:
    name: str
    B: int
    H: int
    N: int
    dtype: str
    gated: bool = False
    decay: Optional[float] = None            # fixed envelope exp(-decay * t)
    decay_loguniform: Optional[tuple] = None  # per-channel decay, log-uniform in [lo, hi]
    squash: Optional[float] = None           # squash threshold lambda
    seed: int = 0
    L: int = 0                                # filter taps (0: the filter is N long)

    @property
    def kind(self):
        return "1d"

    @property
    def taps(self):
        return self.L if self.L else self.N


@dataclasses.dataclass(frozen=True)
class Conv2DSpec:
    name: str
    B: int
    C: int
    S: int                                    # rows (Hs); also the columns unless Ws is set
    dtype: str
    decay: float = 0.05                       # exp(-decay * (|dx| + |dy|)), centred taps
    seed: int = 0
    Ws: int = 0                               # columns of a rectangular image (0: S)

    @property
    def kind(self):
        return "2d"

    @property
    def Hs(self):
        return self.S

    @property
    def cols(self):
        return self.Ws or self.S


@dataclasses.dataclass(frozen=True)
class Conv3DSpec:
    name: str
    B: int
    C: int
    S: int
    dtype: str
    decay: float = 0.1                        # exp(-decay * (|da| + |de| + |df|)), centred taps
    seed: int = 0

    @property
    def kind(self):
        return "3d"


# The five workloads (seed 1000 + i for the i-th, 1-based).
WORKLOADS = {
    "causal_f32_b1_h4_n1024": Conv1DSpec(
        "causal_f32_b1_h4_n1024", 1, 4, 1024, "f32", decay=0.01, squash=0.01, seed=1001),
    "hyena_gated_bf16_b16_h768_n4096": Conv1DSpec(
        "hyena_gated_bf16_b16_h768_n4096", 16, 768, 4096, "bf16", gated=True,
        decay_loguniform=(1e-4, 1e-1), seed=1002),
    "long_f16_b4_h256_n65536": Conv1DSpec(
        "long_f16_b4_h256_n65536", 4, 256, 65536, "f16", decay=1e-4, squash=0.01, seed=1003),
    "very_long_bf16_b1_h64_n2097152": Conv1DSpec(
        "very_long_bf16_b1_h64_n2097152", 1, 64, 2097152, "bf16", decay=1e-6, seed=1004),
    "hyenand_2d_bf16_b8_c256_s128": Conv2DSpec(
        "hyenand_2d_bf16_b8_c256_s128", 8, 256, 128, "bf16", decay=0.05, seed=1005),
    # the 2^21-long shape with a 64-mode state-space filter (chunks with state passing; the
    # modes come from ssm_modes(H, 64, seed + 1))
    "ssm_bf16_b1_h64_n2097152_ns64": Conv1DSpec(
        "ssm_bf16_b1_h64_n2097152_ns64", 1, 64, 2097152, "bf16", decay=1e-6, seed=1008),
    # volumes: the 2D operation one dimension up
    "hyenand_3d_bf16_b4_c128_s32": Conv3DSpec(
        "hyenand_3d_bf16_b4_c128_s32", 4, 128, 32, "bf16", decay=0.1, seed=1007),
    # the 2^21-long shape with a short (4096-tap) filter: the partial convolution
    "partial_bf16_b1_h64_n2097152_l4096": Conv1DSpec(
        "partial_bf16_b1_h64_n2097152_l4096", 1, 64, 2097152, "bf16", decay=1e-3, seed=1006,
        L=4096),
}

# The headline workload the bench times.
HEADLINE = "hyena_gated_bf16_b16_h768_n4096"


def spec_1d(B, H, N, dtype, gated=False, seed=7, decay=None, decay_loguniform=(1e-4, 1e-1),
            squash_lam=None, name=None) -> Conv1DSpec:
    """A custom 1D workload (used for size sweeps in the tests)."""
    if decay is not None:
        decay_loguniform = None
    return Conv1DSpec(name or f"custom_{dtype}_b{B}_h{H}_n{N}", B, H, N, dtype, gated=gated,
                      decay=decay, decay_loguniform=decay_loguniform, squash=squash_lam,
                      seed=seed)


def spec_partial(B, H, N, L, dtype, gated=False, seed=7, decay=1e-3) -> Conv1DSpec:
    """A 1D workload with a short filter of L taps (k is [H, L])."""
    return Conv1DSpec(f"partial_{dtype}_b{B}_h{H}_n{N}_l{L}", B, H, N, dtype, gated=gated,
                      decay=decay, seed=seed, L=L)


def make_1d(spec: Conv1DSpec) -> dict:
    """Draw u, q, v, k, D for a 1D workload (draw order: u, q, v, k_raw, alpha, D); k is
    [H, taps] (taps = N unless the workload has a short filter)."""
    rng = np.random.default_rng(spec.seed)
    B, H, N = spec.B, spec.H, spec.N
    out = {"spec": spec, "dtype": spec.dtype}
    out["u"] = to_storage(rng.standard_normal((B, H, N), dtype=np.float32), spec.dtype)
    if spec.gated:
        out["q"] = to_storage(rng.standard_normal((B, H, N), dtype=np.float32), spec.dtype)
        out["v"] = to_storage(rng.standard_normal((B, H, N), dtype=np.float32), spec.dtype)
    else:
        out["q"] = out["v"] = None
    T = spec.taps
    k = rng.standard_normal((H, T))
    t = np.arange(T, dtype=np.float64)
    if spec.decay_loguniform is not None:
        lo, hi = spec.decay_loguniform
        alpha = np.exp(rng.uniform(math.log(lo), math.log(hi), size=H))
        k *= np.exp(-alpha[:, None] * t[None, :])
    elif spec.decay is not None:
        k *= np.exp(-spec.decay * t)[None, :]
    if spec.squash is not None:
        k = squash(k, spec.squash)
    out["k"] = to_storage(k, spec.dtype)
    out["D"] = to_storage(rng.standard_normal(H), spec.dtype)
    return out


def make_grad_1d(spec: Conv1DSpec) -> np.ndarray:
    """Output gradient dy [B,H,N] ~ N(0,1) in the workload's storage dtype, from its own seeded
    stream (seed + 500000), so the forward draws are unchanged."""
    rng = np.random.default_rng(spec.seed + 500000)
    return to_storage(rng.standard_normal((spec.B, spec.H, spec.N), dtype=np.float32), spec.dtype)


def make_grad_2d(spec: Conv2DSpec) -> np.ndarray:
    """Output gradient dy [B,C,Hs,Ws] ~ N(0,1) in the workload's storage dtype, from its own
    seeded stream (seed + 500000), so the forward draws are unchanged."""
    rng = np.random.default_rng(spec.seed + 500000)
    return to_storage(rng.standard_normal((spec.B, spec.C, spec.Hs, spec.cols), dtype=np.float32), spec.dtype)


def make_2d(spec: Conv2DSpec) -> dict:
    """Draw u, k, D for a 2D workload (draw order: u, k_raw, D)."""
    rng = np.random.default_rng(spec.seed)
    B, C, Hs, Ws = spec.B, spec.C, spec.Hs, spec.cols
    out = {"spec": spec, "dtype": spec.dtype}
    out["u"] = to_storage(rng.standard_normal((B, C, Hs, Ws), dtype=np.float32), spec.dtype)
    k = rng.standard_normal((C, Hs, Ws))
    offh = np.abs(np.arange(Hs, dtype=np.float64) - Hs // 2)
    offw = np.abs(np.arange(Ws, dtype=np.float64) - Ws // 2)
    k *= np.exp(-spec.decay * (offh[:, None] + offw[None, :]))[None]
    out["k"] = to_storage(k, spec.dtype)
    out["D"] = to_storage(rng.standard_normal(C), spec.dtype)
    return out


def ssm_modes(H, NS, seed=0, decay=(1e-4, 1e-1)):
    """Diagonal state-space modes per channel: lam = exp(-a + i theta) with a log-uniform in
    `decay` and theta uniform in [0, pi); W complex Gaussian / sqrt(NS).  complex128 [H, NS]."""
    rng = np.random.default_rng(seed)
    a = np.exp(rng.uniform(math.log(decay[0]), math.log(decay[1]), (H, NS)))
    th = rng.uniform(0.0, math.pi, (H, NS))
    lam = np.exp(-a + 1j * th)
    W = (rng.standard_normal((H, NS)) + 1j * rng.standard_normal((H, NS))) / math.sqrt(NS)
    return lam, W


def butterfly_blocks(N, seed=0):
    """Learned-Butterfly factor blocks for length N (transform M = max(512, next power of two
    >= 2N) = 256 R): complex Gaussian entries of unit variance, so each factor has about the gain
    of its DFT counterpart.  Flat complex64, A1 [R][R], A2, A3, B1, B2 [R][16][16], B3 [R][R]."""
    M = 512
    while M < 2 * N:
        M *= 2
    R = M // 256
    n = 2 * R * R + 4 * 256 * R
    rng = np.random.default_rng(seed)
    z = (rng.standard_normal(n) + 1j * rng.standard_normal(n)) / math.sqrt(2.0)
    return z.astype(np.complex64)


def spec_3d(B, C, S, dtype, seed=7, decay=0.1) -> Conv3DSpec:
    return Conv3DSpec(f"custom3d_{dtype}_b{B}_c{C}_s{S}", B, C, S, dtype, decay=decay, seed=seed)


def make_3d(spec: Conv3DSpec) -> dict:
    """Draw u [B,C,S,S,S], k [C,S,S,S] (centred envelope), D [C] (draw order u, k_raw, D)."""
    rng = np.random.default_rng(spec.seed)
    B, C, S = spec.B, spec.C, spec.S
    out = {"spec": spec, "dtype": spec.dtype}
    out["u"] = to_storage(rng.standard_normal((B, C, S, S, S), dtype=np.float32), spec.dtype)
    k = rng.standard_normal((C, S, S, S))
    r = np.abs(np.arange(S) - S // 2).astype(np.float64)
    env = np.exp(-spec.decay * (r[:, None, None] + r[None, :, None] + r[None, None, :]))
    out["k"] = to_storage(k * env[None], spec.dtype)
    out["D"] = to_storage(rng.standard_normal(C), spec.dtype)
    return out


def sample_points_3d(B, C, S, n=4096, seed=2007):
    """(b,c,i,j,l) voxels: uniform draws plus the corners and faces of the window."""
    rng = np.random.default_rng(seed)
    uni = np.stack([rng.integers(0, B, n), rng.integers(0, C, n)] +
                   [rng.integers(0, S, n) for _ in range(3)], axis=1)
    edge = [0, 1, S // 2 - 1, S // 2, S - 2, S - 1]
    special = [(B - 1, C - 1, i, j, l) for i in edge for j in (0, S - 1) for l in edge]
    return np.ascontiguousarray(np.concatenate([uni, np.asarray(special)], 0).astype(np.int64))


def make(name_or_spec) -> dict:
    spec = WORKLOADS[name_or_spec] if isinstance(name_or_spec, str) else name_or_spec
    return {"1d": make_1d, "2d": make_2d, "3d": make_3d}[spec.kind](spec)


# --------------------------------------------------------------------------------------------
# Sampled output positions
# --------------------------------------------------------------------------------------------

def sample_points_1d(B, H, N, n_uniform=3584, n_struct=512, seed=2000, n_rows=8):
    """(b,h,t) triples: uniform draws plus structured ones on a few seeded rows.

    The structured part covers t in {0, 1, N-2, N-1} and both sides of power-of-two block
    boundaries j*2^m - 1, j*2^m (m >= 8), where a blocked FFT changes blocks.
    """
    rng = np.random.default_rng(seed)
    uni = np.stack([rng.integers(0, B, n_uniform), rng.integers(0, H, n_uniform),
                    rng.integers(0, N, n_uniform)], axis=1)
    rows = np.stack([rng.integers(0, B, n_rows), rng.integers(0, H, n_rows)], axis=1)
    ts = {0, 1, max(N - 2, 0), N - 1}
    m = 8
    while (1 << m) < N:
        step = 1 << m
        for j in rng.integers(1, max(N // step, 1) + 1, 3):
            for t in (j * step - 1, j * step):
                if 0 <= t < N:
                    ts.add(int(t))
        m += 1
    ts = sorted(ts)
    struct = []
    for i in range(n_struct):
        b, h = rows[i % n_rows]
        struct.append((b, h, ts[(i // n_rows) % len(ts)] if i < n_rows * len(ts)
                       else int(rng.integers(0, N))))
    pts = np.concatenate([uni, np.asarray(struct, np.int64).reshape(-1, 3)], axis=0)
    return np.ascontiguousarray(pts.astype(np.int64))


def sample_points_2d(B, C, S, n=4096, seed=2005):
    """(b,c,i,j) quadruples: uniform draws plus every corner and centre pixel of a few images."""
    rng = np.random.default_rng(seed)
    uni = np.stack([rng.integers(0, B, n - 64), rng.integers(0, C, n - 64),
                    rng.integers(0, S, n - 64), rng.integers(0, S, n - 64)], axis=1)
    special = []
    for r in range(8):
        b, c = int(rng.integers(0, B)), int(rng.integers(0, C))
        for (i, j) in ((0, 0), (0, S - 1), (S - 1, 0), (S - 1, S - 1),
                       (S // 2, S // 2), (S // 2 - 1, S // 2), (0, S // 2), (S - 1, S // 2)):
            special.append((b, c, i, j))
    return np.ascontiguousarray(np.concatenate([uni, np.asarray(special)], 0).astype(np.int64))

"""GPU parity: the HIP path through the C ABI against the float64 CPU oracle.

Tolerance (stated with the workloads): max relative L2 error 1e-4 for fp32 inputs, 2e-2 for
bf16/fp16 inputs, per fully checked (b,h) row; pooled over the sampled positions where the
oracle samples.  Any non-finite output fails.
"""
import numpy as np
import pytest

import oracle
from fft_long_convolution_amd import workloads as wl
from tests.gpu_util import DT_ORACLE, TOL, from_dev, rel_l2, rel_l2_rows, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lc():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fft_long_convolution_amd import lconv
    lconv.load()
    return lconv


def run_1d(lc, d):
    """Filter FFT + forward through the ABI; returns y as float64 numpy."""
    import torch
    dt = d["dtype"]
    k = to_dev(d["k"], dt)
    u, q, v, D = (to_dev(d[x], dt) for x in ("u", "q", "v", "D"))
    kf = lc.filter_fft(k)
    y = lc.fftconv(u, kf, D, q=q, v=v)
    torch.cuda.synchronize()
    return from_dev(y, dt), (u, kf, D, q, v)


def oracle_rows(d, rows, nthreads):
    return oracle.conv1d_rows(d["u"], d["k"], d["D"], rows, q=d["q"], v=d["v"],
                              dt=DT_ORACLE[d["dtype"]], nthreads=nthreads)


SWEEP_N = [8, 64, 120, 256, 1000, 1024, 2048, 4096, 8192, 16384]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("N", SWEEP_N)
@pytest.mark.parametrize("B,gated", [(1, False), (3, True), (4, False)])
def test_sweep_full_rows(lc, nthreads, dtype, N, B, gated):
    H = 3
    spec = wl.spec_1d(B, H, N, dtype, gated=gated, seed=100 + N + B)
    say(f"[sweep] dtype={dtype} B={B} H={H} N={N} gated={gated} seed={spec.seed}")
    d = wl.make(spec)
    y, _ = run_1d(lc, d)
    assert np.all(np.isfinite(y))
    rows = [(b, h) for b in range(B) for h in range(H)]
    ref = oracle_rows(d, rows, nthreads).reshape(B, H, N)
    err = rel_l2_rows(y, ref).max()
    say(f"   max rel L2 = {err:.3e} (tol {TOL[dtype]})")
    assert err <= TOL[dtype]


def test_workload_causal_f32(lc, nthreads):
    d = wl.make("causal_f32_b1_h4_n1024")
    say("[workload] causal_f32_b1_h4_n1024")
    y, _ = run_1d(lc, d)
    ref = oracle_rows(d, [(0, h) for h in range(4)], nthreads).reshape(1, 4, 1024)
    err = rel_l2_rows(y, ref).max()
    say(f"   max rel L2 = {err:.3e}")
    assert err <= 1e-4


def test_workload_hyena_gated_bf16(lc, nthreads):
    """B16 H768 N4096: every one of the 12,288 (b,h) rows against the oracle, plus the 4096
    sampled positions (pooled) that the larger workloads use."""
    name = "hyena_gated_bf16_b16_h768_n4096"
    d = wl.make(name)
    say(f"[workload] {name}")
    y, _ = run_1d(lc, d)
    assert np.all(np.isfinite(y))
    rows = [(b, h) for b in range(16) for h in range(768)]
    ref = oracle_rows(d, rows, nthreads).reshape(16, 768, 4096)
    per_row = rel_l2_rows(y, ref)
    worst = np.unravel_index(int(np.argmax(per_row)), per_row.shape)
    max_abs = float(np.max(np.abs(y - ref)))
    pts = wl.sample_points_1d(16, 768, 4096, seed=2002)
    refp = oracle.conv1d_points(d["u"], d["k"], d["D"], pts, q=d["q"], v=d["v"],
                                dt=oracle.DT_BF16, nthreads=nthreads)
    err_pts = rel_l2(y[pts[:, 0], pts[:, 1], pts[:, 2]], refp)
    say(f"   all 12288 rows: max rel L2 = {per_row.max():.3e} at (b,h)={tuple(int(i) for i in worst)}, "
        f"median {np.median(per_row):.3e}, max abs err {max_abs:.3e}; sampled pooled rel L2 = {err_pts:.3e}")
    assert per_row.max() <= 2e-2 and err_pts <= 2e-2


# The M = 8192 pipelined kernel (N = 4096, 16-bit) gives each workgroup a run of items (batch
# pairs); its first two and last two items take guarded copies of the loop body.  On 256 compute
# units these shapes give 2, 3, 4, 5 and 9 items per workgroup, a last workgroup with fewer
# items, odd batches (a pair repeating its row) and channel changes inside a workgroup's run.
PIPELINE_SHAPES = [(2, 300), (2, 301), (3, 300), (2, 1000), (5, 400), (6, 700)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("B,H", PIPELINE_SHAPES)
def test_pipelined_items_per_workgroup(lc, nthreads, dtype, B, H):
    spec = wl.spec_1d(B, H, 4096, dtype, gated=True, seed=3000 + 7 * B + H)
    say(f"[pipeline] dtype={dtype} B={B} H={H} N=4096 gated seed={spec.seed}")
    d = wl.make(spec)
    y, _ = run_1d(lc, d)
    assert np.all(np.isfinite(y))
    rows = [(b, h) for b in range(B) for h in range(H)]
    ref = oracle_rows(d, rows, nthreads).reshape(B, H, 4096)
    per_row = rel_l2_rows(y, ref)
    worst = np.unravel_index(int(np.argmax(per_row)), per_row.shape)
    say(f"   all {B * H} rows: max rel L2 = {per_row.max():.3e} at (b,h)={tuple(int(i) for i in worst)}")
    assert per_row.max() <= TOL[dtype]


def _sampled_long(lc, name, nthreads, n_rows_full=0):
    d = wl.make(name)
    spec = d["spec"]
    say(f"[workload] {name}")
    y, _ = run_1d(lc, d)
    assert np.all(np.isfinite(y))
    pts = wl.sample_points_1d(spec.B, spec.H, spec.N, seed=spec.seed + 1000)
    refp = oracle.conv1d_points(d["u"], d["k"], d["D"], pts, q=d["q"], v=d["v"],
                                dt=DT_ORACLE[spec.dtype], nthreads=nthreads)
    err = rel_l2(y[pts[:, 0], pts[:, 1], pts[:, 2]], refp)
    say(f"   sampled pooled rel L2 = {err:.3e}")
    assert err <= TOL[spec.dtype]
    if n_rows_full:
        rng = np.random.default_rng(spec.seed + 2000)
        rows = np.stack([rng.integers(0, spec.B, n_rows_full), rng.integers(0, spec.H, n_rows_full)], 1)
        ref = oracle_rows(d, rows, nthreads)
        e2 = rel_l2_rows(y[rows[:, 0], rows[:, 1]], ref).max()
        say(f"   full rows max rel L2 = {e2:.3e}")
        assert e2 <= TOL[spec.dtype]


def test_workload_long_f16(lc, nthreads):
    _sampled_long(lc, "long_f16_b4_h256_n65536", nthreads, n_rows_full=4)


def test_workload_very_long_bf16(lc, nthreads):
    _sampled_long(lc, "very_long_bf16_b1_h64_n2097152", nthreads)


def test_deterministic(lc):
    import torch
    d = wl.make(wl.spec_1d(6, 5, 4096, "bf16", gated=True, seed=77))
    say("[determinism] bf16 B6 H5 N4096 gated")
    _, (u, kf, D, q, v) = run_1d(lc, d)
    y1 = lc.fftconv(u, kf, D, q=q, v=v)
    y2 = lc.fftconv(u, kf, D, q=q, v=v)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_empty_and_stream(lc):
    import torch
    u = torch.zeros((0, 3, 64), dtype=torch.bfloat16, device="cuda")
    kf = lc.filter_fft(torch.zeros((3, 64), dtype=torch.bfloat16, device="cuda"))
    D = torch.zeros(3, dtype=torch.bfloat16, device="cuda")
    y = lc.fftconv(u, kf, D)
    assert y.shape == (0, 3, 64)
    # a non-default stream gives the same result
    d = wl.make(wl.spec_1d(2, 2, 512, "bf16", seed=5))
    y0, (u, kf, D, q, v) = run_1d(lc, d)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y1 = lc.fftconv(u, kf, D, stream=s)
    s.synchronize()
    assert np.array_equal(from_dev(y1, "bf16"), y0)


RAGGED_N = [1, 7, 13, 100, 1001, 4095, 4097]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N", RAGGED_N)
@pytest.mark.parametrize("B,gated", [(1, False), (3, True)])
def test_ragged_lengths_full_rows(lc, nthreads, dtype, N, B, gated):
    """N not a multiple of 8: rows staged zero-padded through the workspace."""
    H = 2
    spec = wl.spec_1d(B, H, N, dtype, gated=gated, seed=1300 + N + B)
    say(f"[ragged] dtype={dtype} B={B} H={H} N={N} gated={gated} seed={spec.seed}")
    d = wl.make(spec)
    y, _ = run_1d(lc, d)
    assert y.shape == (B, H, N) and np.all(np.isfinite(y))
    rows = [(b, h) for b in range(B) for h in range(H)]
    ref = oracle_rows(d, rows, nthreads).reshape(B, H, N)
    err = rel_l2_rows(y, ref).max()
    say(f"   max rel L2 = {err:.3e} (tol {TOL[dtype]})")
    assert err <= TOL[dtype]


def test_ragged_multipass_sampled(lc, nthreads):
    """A ragged length past one workgroup (multi-pass path), sampled."""
    B, H, N = 3, 2, 65537
    spec = wl.spec_1d(B, H, N, "bf16", gated=True, seed=1399, decay=1e-4)
    say(f"[ragged long] B={B} H={H} N={N} seed={spec.seed}")
    d = wl.make(spec)
    y, _ = run_1d(lc, d)
    pts = wl.sample_points_1d(B, H, N, seed=2400)
    ref = oracle.conv1d_points(d["u"], d["k"], d["D"], pts, q=d["q"], v=d["v"], dt=oracle.DT_BF16,
                               nthreads=nthreads)
    got = y[pts[:, 0], pts[:, 1], pts[:, 2]]
    err = rel_l2(got, ref)
    say(f"   pooled rel L2 over {len(pts)} positions = {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= TOL["bf16"]

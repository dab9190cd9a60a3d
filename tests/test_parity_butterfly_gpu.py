"""GPU parity of the learned-Butterfly convolution: lconv_butterfly_tables, lconv_butterfly_filter
and lconv_butterfly_fwd through the C ABI against the float64 oracle (oracle.butterfly, pinned in
tests/test_oracle_butterfly.py), on every output of every row.

The factor blocks are seeded complex Gaussians (workloads.butterfly_blocks), the same fp32 values
for both sides; the kernel rounds them to its compute type as it does the DFT's own blocks.
Tolerance as for the forward: max relative L2 error per row 1e-4 (fp32), 2e-2 (bf16 / fp16).
"""
import numpy as np
import pytest

from oracle import butterfly as bf
from fft_long_convolution_amd import workloads as wl
from tests.gpu_util import DT_ORACLE, TOL, from_dev, rel_l2_rows, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lc():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fft_long_convolution_amd import lconv
    lconv.load()
    return lconv


def _torch_dtype(dtype):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


# (B, H, N, gates): every transform length M = 512 .. 8192 (R = 2 .. 32), odd and even batches,
# a length that does not fill the half transform
CASES = [(3, 2, 256, "qv"), (2, 3, 1000, "q"), (1, 2, 1024, ""), (4, 2, 2048, "v"), (3, 2, 4096, "qv"),
         (2, 2, 4000, "")]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("B,H,N,gates", CASES)
def test_butterfly_full_rows(lc, dtype, B, H, N, gates):
    import torch
    spec = wl.spec_1d(B, H, N, dtype, gated=True, seed=1300 + N + B)
    d = wl.make(spec)
    q = d["q"] if "q" in gates else None
    v = d["v"] if "v" in gates else None
    blocks = wl.butterfly_blocks(N, seed=77 + N)
    say(f"[butterfly] dtype={dtype} B={B} H={H} N={N} gates={gates!r} seed={spec.seed} blocks_seed={77 + N}")
    tables = lc.butterfly_tables(torch.from_numpy(blocks).cuda(), N, _torch_dtype(dtype))
    kf = lc.butterfly_filter(to_dev(d["k"], dtype), tables)
    u_d, D_d, q_d, v_d = (to_dev(x, dtype) for x in (d["u"], d["D"], q, v))
    y = lc.butterfly(u_d, kf, D_d, tables, q=q_d, v=v_d)
    torch.cuda.synchronize()
    got = from_dev(y, dtype).reshape(B * H, N)
    ref = bf.butterfly_conv(d["u"], d["k"], d["D"], blocks, q=q, v=v, dt=DT_ORACLE[dtype]).reshape(B * H, N)
    assert np.all(np.isfinite(got))
    err = float(rel_l2_rows(got, ref).max())
    say(f"   max rel L2 = {err:.3e} (tol {TOL[dtype]})")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_dft_blocks_reduce_to_the_fft_convolution(lc, dtype):
    """With the DFT's own blocks the learned path is the ordinary convolution call."""
    import torch
    B, H, N = 3, 4, 4096
    spec = wl.spec_1d(B, H, N, dtype, gated=True, seed=1401)
    d = wl.make(spec)
    bl = bf.dft_blocks(8192)
    flat = np.concatenate([bl[n].ravel() for n in ("A1", "A2", "A3", "B1", "B2", "B3")]).astype(np.complex64)
    say(f"[butterfly dft] dtype={dtype} seed={spec.seed}")
    tables = lc.butterfly_tables(torch.from_numpy(flat).cuda(), N, _torch_dtype(dtype))
    u, q, v, D, k = (to_dev(d[x], dtype) for x in ("u", "q", "v", "D", "k"))
    yb = lc.butterfly(u, lc.butterfly_filter(k, tables), D, tables, q=q, v=v)
    yd = lc.fftconv(u, lc.filter_fft(k), D, q=q, v=v)
    torch.cuda.synchronize()
    err = float(rel_l2_rows(from_dev(yb, dtype).reshape(B * H, N), from_dev(yd, dtype).reshape(B * H, N)).max())
    say(f"   max rel L2 between the two calls = {err:.3e}")
    assert err <= (1e-4 if dtype == "f32" else 2e-2)


def test_butterfly_deterministic(lc):
    import torch
    B, H, N = 2, 3, 2048
    spec = wl.spec_1d(B, H, N, "bf16", gated=True, seed=1402)
    d = wl.make(spec)
    blocks = torch.from_numpy(wl.butterfly_blocks(N, seed=5)).cuda()
    say(f"[butterfly determinism] seed={spec.seed}")
    outs = []
    for _ in range(2):
        tables = lc.butterfly_tables(blocks, N, torch.bfloat16)
        kf = lc.butterfly_filter(to_dev(d["k"], "bf16"), tables)
        outs.append(lc.butterfly(to_dev(d["u"], "bf16"), kf, to_dev(d["D"], "bf16"), tables,
                                 q=to_dev(d["q"], "bf16"), v=to_dev(d["v"], "bf16")))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])

"""GPU parity of the training pair lconv_fftconv_fwd_save + lconv_fftconv_bwd_saved.

* y from the saving forward equals lconv_fftconv_fwd's y bit for bit (the same chain), and the
  saved pre-gate output c matches the float64 oracle's convolution without the v gate.
* The saved-output gradient gives du, dq, dk, dD identical to lconv_fftconv_bwd (the same
  launches) and dv = dy * c within the usual tolerance of the oracle's dv.
Tolerances as for the forward: max relative L2 1e-4 (fp32), 2e-2 (bf16 / fp16) per row.
"""
import numpy as np
import pytest

import oracle
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


# (B, H, N, gates): the pipelined kernel (N = 4096, 16-bit), the generic kernels, odd batches
CASES = [(2, 3, 4096, "qv"), (3, 2, 4096, "v"), (1, 2, 1000, "qv"), (2, 2, 256, "q"), (3, 1, 64, "")]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("B,H,N,gates", CASES)
def test_save_and_saved_gradient(lc, nthreads, dtype, B, H, N, gates):
    import torch
    spec = wl.spec_1d(B, H, N, dtype, gated=True, seed=3100 + N + B)
    say(f"[save] dtype={dtype} B={B} H={H} N={N} gates={gates!r} seed={spec.seed}")
    d = wl.make(spec)
    dy = wl.make_grad_1d(spec)
    q = d["q"] if "q" in gates else None
    v = d["v"] if "v" in gates else None
    dev = lambda a: to_dev(a, dtype)
    u_d, D_d, q_d, v_d, dy_d = dev(d["u"]), dev(d["D"]), dev(q), dev(v), dev(dy)
    kf = lc.filter_fft(dev(d["k"]))
    y_ref = lc.fftconv(u_d, kf, D_d, q=q_d, v=v_d)
    y, c = lc.fftconv_save(u_d, kf, D_d, q=q_d, v=v_d)
    g_plain = lc.fftconv_bwd(dy_d, u_d, kf, D_d, q=q_d, v=v_d)
    g_saved = lc.fftconv_bwd(dy_d, u_d, kf, D_d, q=q_d, v=v_d, c=c)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref), "the saving forward must give the same y"
    rows = [(b, h) for b in range(B) for h in range(H)]
    c_ref = oracle.conv1d_rows(d["u"], d["k"], d["D"], rows, q=q, v=None, dt=DT_ORACLE[dtype],
                               nthreads=nthreads).reshape(B, H, N)
    cg = from_dev(c, dtype)
    err_c = float(rel_l2_rows(cg, c_ref).max())
    say(f"   c max rel L2 = {err_c:.3e}")
    assert np.all(np.isfinite(cg)) and err_c <= TOL[dtype]
    names = ["du", "dq", "dv", "dk", "dD"]
    for name, a, b in zip(names, g_plain, g_saved):
        if a is None:
            assert b is None, name
            continue
        if name != "dv":
            assert torch.equal(a, b), name
    if v is not None:
        _, _, r_dv = oracle.conv1d_bwd_rows(d["u"], d["k"], d["D"], dy, rows, q=q, v=v,
                                            dt=DT_ORACLE[dtype], nthreads=nthreads)
        dvg = from_dev(g_saved[2], dtype).reshape(B * H, N)
        err_dv = float(rel_l2_rows(dvg, r_dv).max())
        say(f"   dv max rel L2 = {err_dv:.3e}")
        assert np.all(np.isfinite(dvg)) and err_dv <= TOL[dtype]

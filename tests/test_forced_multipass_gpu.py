"""The multi-pass path forced at lengths one workgroup would take (LCONV_FORCE_PATH=multipass:
every length on the column/row/column passes with at least two columns), against the oracle on
full rows, so the pass boundaries are checked where the oracle is cheap.  The switch is read once
per process, so the check runs in a child process with the variable set; LCONV_LOG=1 makes the
child's library print the plans it ran, which must say 'forced'."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
import numpy as np
import torch
sys.path.insert(0, ROOT)
import oracle
from fft_long_convolution_amd import lconv, workloads as wl
from tests.gpu_util import DT_ORACLE, TOL, from_dev, rel_l2_rows, to_dev
lconv.load()
worst = 0.0
for dt in ("bf16", "f32"):
    for N, B in ((1024, 3), (4096, 2), (1000, 1), (64, 2)):
        spec = wl.spec_1d(B, 2, N, dt, gated=True, seed=950 + N + B)
        d = wl.make(spec)
        u, q, v, k, D = (to_dev(d[x], dt) for x in ("u", "q", "v", "k", "D"))
        kf = lconv.filter_fft(k)
        y = from_dev(lconv.fftconv(u, kf, D, q=q, v=v), dt)
        rows = [(b, h) for b in range(B) for h in range(2)]
        ref = oracle.conv1d_rows(d["u"], d["k"], d["D"], rows, q=d["q"], v=d["v"], dt=DT_ORACLE[dt]).reshape(B, 2, N)
        err = float(rel_l2_rows(y, ref).max())
        print(f"forced multi-pass {dt} B={B} N={N}: max rel L2 {err:.3e}", flush=True)
        assert np.all(np.isfinite(y)) and err <= TOL[dt], (dt, N, err)
        if N % 8 == 0:
            dy = wl.make_grad_1d(spec)
            du, dq, dv, dk, dD = lconv.fftconv_bwd(to_dev(dy, dt), u, kf, D, q=q, v=v)
            r_du, r_dq, r_dv = oracle.conv1d_bwd_rows(d["u"], d["k"], d["D"], dy, rows, q=d["q"], v=d["v"],
                                                      dt=DT_ORACLE[dt])
            r_dk, _ = oracle.conv1d_bwd_dk(d["u"], dy, [0, 1], q=d["q"], v=d["v"], dt=DT_ORACLE[dt])
            e = max(float(rel_l2_rows(from_dev(du, dt).reshape(-1, N), r_du).max()),
                    float(rel_l2_rows(from_dev(dq, dt).reshape(-1, N), r_dq).max()),
                    float(rel_l2_rows(from_dev(dv, dt).reshape(-1, N), r_dv).max()),
                    float(rel_l2_rows(dk.cpu().numpy().astype(np.float64), r_dk).max()))
            print(f"forced multi-pass gradient {dt} B={B} N={N}: max rel L2 {e:.3e}", flush=True)
            assert e <= TOL[dt], (dt, N, e)
print("FORCED_OK")
"""


def test_forced_multipass_against_oracle():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    env = dict(os.environ, LCONV_FORCE_PATH="multipass", LCONV_LOG="1")
    r = subprocess.run([sys.executable, "-u", "-c", f"ROOT = {ROOT!r}\n" + CHILD], env=env, cwd=ROOT,
                       capture_output=True, text=True, timeout=240)
    print(r.stdout)
    print(r.stderr[-4000:])
    assert r.returncode == 0 and "FORCED_OK" in r.stdout
    assert "forced" in r.stderr and "multi-pass" in r.stderr

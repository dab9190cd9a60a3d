"""Pins for the gradient oracle (oracle.conv1d_bwd_rows / conv1d_bwd_dk), CPU only.

The output y = v (k * x + D x), x = q u, is linear in each of u, q, v and (k, D) separately, so
for an output gradient gy and any direction delta:

    <y(theta + delta) - y(theta), gy> = <d_theta, delta>        (theta = u, q, v or (k, D))

exactly in real arithmetic.  Checked in float64 with random directions (forward values from the
independent forward oracle), against float64 torch autograd of a convolution written with
torch.nn.functional.conv1d, and by exact integer arithmetic on a tiny case.  Each planted
mistake below (a wrong lag direction, an off-by-one lag, a dropped skip term, a swapped gate,
a reversed filter gradient) fails at least one pin.
"""
import numpy as np
import pytest

import oracle


def _draw(B, H, N, seed, gated=True):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    u, gy = f(B, H, N), f(B, H, N)
    q, v = (f(B, H, N), f(B, H, N)) if gated else (None, None)
    k, D = f(H, N), f(H)
    return u, q, v, k, D, gy


def _fwd(u, q, v, k, D):
    B, H, N = u.shape
    rows = [(b, h) for b in range(B) for h in range(H)]
    return oracle.conv1d_rows(u, k, D, rows, q=q, v=v).reshape(B, H, N)


def _grads(u, q, v, k, D, gy):
    B, H, N = u.shape
    rows = [(b, h) for b in range(B) for h in range(H)]
    du, dq, dv = oracle.conv1d_bwd_rows(u, k, D, gy, rows, q=q, v=v)
    dk, dD = oracle.conv1d_bwd_dk(u, gy, list(range(H)), q=q, v=v)
    r = lambda a: None if a is None else a.reshape(B, H, N)
    return {"u": r(du), "q": r(dq), "v": r(dv), "k": dk, "D": dD}


# ---- reference implementations used as pins (and their planted mistakes) --------------------

def grads_numpy(u, q, v, k, D, gy, mutant=None):
    """The chain rule written out with numpy (same formulas as the C oracle), optionally with
    one planted mistake."""
    u, k, D, gy = (np.asarray(a, np.float64) for a in (u, k, D, gy))
    B, H, N = u.shape
    q = np.ones_like(u) if q is None else np.asarray(q, np.float64)
    v = np.ones_like(u) if v is None else np.asarray(v, np.float64)
    x, ds = q * u, gy * v
    du, dq, dv = np.zeros_like(u), np.zeros_like(u), np.zeros_like(u)
    dk, dD = np.zeros((H, N)), np.zeros(H)
    for b in range(B):
        for h in range(H):
            kk = k[h]
            if mutant == "k_reversed":
                kk = kk[::-1]
            # dx[t] = sum_{tau >= t} k[tau - t] ds[tau] + D ds[t]
            full = np.correlate(ds[b, h], kk, mode="full")  # full[N-1+j] = sum_t ds[t+j] kk[t]
            dx = full[N - 1:] if mutant != "causal_dx" else np.convolve(ds[b, h], kk)[:N]
            if mutant == "lag_shift":
                dx = np.concatenate([dx[1:], [0.0]])
            skip = D[h] * ds[b, h] if mutant != "no_skip" else 0.0
            dx = dx + skip
            du[b, h] = q[b, h] * dx
            dq[b, h] = (q if mutant == "gate_swap" else u)[b, h] * dx
            s = np.convolve(x[b, h], k[h])[:N] + D[h] * x[b, h]
            dv[b, h] = gy[b, h] * s
            c = np.correlate(ds[b, h], x[b, h], mode="full")[N - 1:]  # c[tau] = sum ds[t] x[t-tau]
            dk[h] += c if mutant != "dk_reversed" else c[::-1]
            dD[h] += c[0]
    return {"u": du, "q": dq, "v": dv, "k": dk, "D": dD}


def pin_directional(gfun, B=2, H=2, N=24, seed=3):
    """<y(theta + delta) - y(theta), gy> == <d_theta, delta> for random delta, each argument."""
    u, q, v, k, D, gy = _draw(B, H, N, seed)
    g = gfun(u, q, v, k, D, gy)
    y0 = _fwd(u, q, v, k, D)
    rng = np.random.default_rng(seed + 1)
    # theta + delta is rounded to float32 storage; the step actually taken is measured after
    # rounding, so the identity holds to float64 rounding of the sums
    d = lambda *s: rng.integers(-8, 9, s) / 64.0
    step = lambda a, dl: ((a + dl).astype(np.float32),
                          (a + dl).astype(np.float32).astype(np.float64) - a.astype(np.float64))
    ok = True
    for name in ("u", "q", "v"):
        args = dict(u=u, q=q, v=v, k=k, D=D)
        args[name], delta = step(args[name], d(B, H, N))
        y1 = _fwd(args["u"], args["q"], args["v"], k, D)
        lhs = float(((y1 - y0) * gy).sum())
        rhs = float((g[name] * delta).sum())
        ok &= abs(lhs - rhs) <= 1e-9 * (1 + abs(lhs))
    k1, dk = step(k, d(H, N))
    D1, dD = step(D, d(H))
    y1 = _fwd(u, q, v, k1, D1)
    lhs = float(((y1 - y0) * gy).sum())
    rhs = float((g["k"] * dk).sum() + (g["D"] * dD).sum())
    ok &= abs(lhs - rhs) <= 1e-9 * (1 + abs(lhs))
    # dk and dD separately (catches an error that trades one for the other)
    y2 = _fwd(u, q, v, k, D1)
    ok &= abs(float(((y2 - y0) * gy).sum()) - float((g["D"] * dD).sum())) <= 1e-9 * (1 + abs(lhs))
    return ok


def pin_torch(gfun, B=2, H=3, N=20, seed=5):
    """Float64 torch autograd of the same operator written with conv1d."""
    torch = pytest.importorskip("torch")
    u, q, v, k, D, gy = _draw(B, H, N, seed)
    T = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    tu, tq, tv, tk, tD = T(u), T(q), T(v), T(k), T(D)
    x = tq * tu
    # causal conv: pad left by N-1, flip the kernel for conv1d (which is a correlation)
    xp = torch.nn.functional.pad(x, (N - 1, 0))
    s = torch.nn.functional.conv1d(xp, tk.flip(-1).unsqueeze(1), groups=H) + tD[None, :, None] * x
    y = tv * s
    (y * torch.tensor(gy, dtype=torch.float64)).sum().backward()
    g = gfun(u, q, v, k, D, gy)
    ref = {"u": tu.grad, "q": tq.grad, "v": tv.grad, "k": tk.grad, "D": tD.grad}
    return all(np.allclose(g[n], ref[n].numpy(), rtol=1e-10, atol=1e-10) for n in ref)


def pin_integer(gfun):
    """Small integers: every intermediate is exact in float64; compare with Python ints."""
    B, H, N = 2, 1, 9
    rng = np.random.default_rng(11)
    I = lambda *s: rng.integers(-3, 4, s).astype(np.float32)
    u, q, v, gy, k, D = I(B, H, N), I(B, H, N), I(B, H, N), I(B, H, N), I(H, N), I(H)
    g = gfun(u, q, v, k, D, gy)
    ok = True
    for b in range(B):
        ds = [int(gy[b, 0, t]) * int(v[b, 0, t]) for t in range(N)]
        x = [int(q[b, 0, t]) * int(u[b, 0, t]) for t in range(N)]
        for t in range(N):
            dx = sum(int(k[0, tau - t]) * ds[tau] for tau in range(t, N)) + int(D[0]) * ds[t]
            ok &= g["u"][b, 0, t] == int(q[b, 0, t]) * dx
            ok &= g["q"][b, 0, t] == int(u[b, 0, t]) * dx
    dk = [sum(int(gy[b, 0, t]) * int(v[b, 0, t]) * int(q[b, 0, t - tau]) * int(u[b, 0, t - tau])
              for b in range(B) for t in range(tau, N)) for tau in range(N)]
    ok &= all(g["k"][0, tau] == dk[tau] for tau in range(N)) and g["D"][0] == dk[0]
    return bool(ok)


PINS = [pin_directional, pin_torch, pin_integer]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_gradients_pass_pins(pin):
    assert pin(lambda *a: _grads(*a))


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_numpy_chain_rule_passes_pins(pin):
    assert pin(lambda *a: grads_numpy(*a))


@pytest.mark.parametrize("mutant", ["causal_dx", "lag_shift", "no_skip", "gate_swap",
                                    "k_reversed", "dk_reversed"])
def test_planted_mistakes_fail_a_pin(mutant):
    fails = [not pin(lambda *a: grads_numpy(*a, mutant=mutant)) for pin in PINS]
    assert any(fails), mutant


def test_oracle_equals_numpy_chain_rule():
    u, q, v, k, D, gy = _draw(3, 2, 33, 21)
    g, r = _grads(u, q, v, k, D, gy), grads_numpy(u, q, v, k, D, gy)
    for n in g:
        assert np.allclose(g[n], r[n], rtol=1e-12, atol=1e-9), n


def test_ungated_gradients():
    """Without gates du = dx and dq, dv are not produced."""
    u, _, _, k, D, gy = _draw(2, 2, 17, 8, gated=False)
    rows = [(b, h) for b in range(2) for h in range(2)]
    du, dq, dv = oracle.conv1d_bwd_rows(u, k, D, gy, rows)
    assert dq is None and dv is None
    r = grads_numpy(u, None, None, k, D, gy)
    assert np.allclose(du.reshape(2, 2, 17), r["u"], rtol=1e-12, atol=1e-9)
    dk, dD = oracle.conv1d_bwd_dk(u, gy, [0, 1])
    assert np.allclose(dk, r["k"], rtol=1e-12, atol=1e-9) and np.allclose(dD, r["D"])


def test_bwd_rejects_bad_arguments():
    u, q, v, k, D, gy = _draw(1, 1, 8, 1)
    with pytest.raises(ValueError):
        oracle.conv1d_bwd_rows(u, k, D, gy, [(1, 0)], q=q, v=v)
    with pytest.raises(ValueError):
        oracle.conv1d_bwd_dk(u, gy, [3], q=q, v=v)


@pytest.mark.parametrize("gated", [True, False])
def test_points_match_rows_bitwise(gated):
    """The single-position gradients sum exactly as the row and channel versions do."""
    B, H, N = 3, 2, 64
    u, q, v, k, D, gy = _draw(B, H, N, seed=91, gated=gated)
    rows = [(b, h) for b in range(B) for h in range(H)]
    du, dq, dv = oracle.conv1d_bwd_rows(u, k, D, gy, rows, q=q, v=v)
    dk, dD = oracle.conv1d_bwd_dk(u, gy, list(range(H)), q=q, v=v)
    rng = np.random.default_rng(5)
    pts = np.stack([rng.integers(0, B, 200), rng.integers(0, H, 200), rng.integers(0, N, 200)], 1)
    pts[:4] = [(0, 0, 0), (B - 1, H - 1, N - 1), (1, 0, N - 2), (2, 1, 1)]
    pu, pq, pv = oracle.conv1d_bwd_points(u, k, D, gy, pts, q=q, v=v)
    idx = pts[:, 0] * H + pts[:, 1]
    assert np.array_equal(pu, du[idx, pts[:, 2]])
    if gated:
        assert np.array_equal(pq, dq[idx, pts[:, 2]]) and np.array_equal(pv, dv[idx, pts[:, 2]])
    else:
        assert pq is None and pv is None
    kp = np.stack([rng.integers(0, H, 100), rng.integers(0, N, 100)], 1)
    kp[:2] = [(0, 0), (H - 1, N - 1)]
    pk = oracle.conv1d_bwd_dk_points(u, gy, kp, q=q, v=v)
    assert np.array_equal(pk, dk[kp[:, 0], kp[:, 1]])
    assert np.array_equal(oracle.conv1d_bwd_dk_points(u, gy, [(h, 0) for h in range(H)], q=q, v=v), dD)

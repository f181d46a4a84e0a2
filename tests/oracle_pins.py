"""Pins for the fp64 oracle: checks against facts fixed outside the oracle.

Each ``pin_*`` takes a loaded oracle (``oracle.Oracle``) and raises
``AssertionError`` if the oracle disagrees with a closed form, a brute-force
evaluation written a different way, an invariant, or the hand-worked example.
The same pins are run against deliberately broken builds of the oracle
(``test_oracle_mutants.py``) to show that a plausible mistake is caught.

The independent formulas used here:
  * softplus via ``numpy.logaddexp(0, x)``; the sigmoid via 0.5 (1 + tanh(z/2));
  * the unrolled (dual, attention-like) form of the scan, y_k = sum_{j<=k}
    C_k (prod_{l=j+1..k} Abar_l) Bbar_j u_j ("Understanding Mamba",
    aiattnstudio.link, sections 6.1 and 12), with the products of Abar written
    as exp(A (S_k - S_j)), S = cumulative sum of Delta;
  * the LTI convolution kernel K = (C Bbar, C Abar Bbar, C Abar^2 Bbar, ...)
    (hnwysp.cn Mamba slides, section 2.1), with Abar^k = exp(k Delta A).
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# independent reference pieces
# ----------------------------------------------------------------------------

def ref_softplus(x):
    return np.logaddexp(0.0, x)


def ref_silu(z):
    return z * 0.5 * (1.0 + np.tanh(0.5 * np.asarray(z, dtype=np.float64)))


def brute_force(u, delta, A, B, C, D=None, z=None, bias=None, h0=None):
    """O(L^2) evaluation of the unrolled form, independent of the recurrence."""
    batch, L, Dn = u.shape
    N = A.shape[1]
    y = np.zeros_like(u)
    h_last = np.zeros((batch, Dn, N))
    bias_v = np.zeros(Dn) if bias is None else bias
    for b in range(batch):
        for d in range(Dn):
            dt = ref_softplus(delta[b, :, d] + bias_v[d])          # (L,)
            S = np.cumsum(dt)                                     # S_t
            a = A[d]                                              # (N,)
            # G[t, j, n] = exp(A_n (S_t - S_j)) for j <= t
            diff = S[:, None] - S[None, :]
            mask = np.tril(np.ones((L, L), dtype=bool))
            G = np.exp(np.where(mask, diff, 0.0)[:, :, None] * a[None, None, :])
            G = G * mask[:, :, None]
            src = dt[:, None] * B[b] * u[b, :, d][:, None]        # Bbar_j u_j (L, N)
            h_all = np.einsum("tjn,jn->tn", G, src)                # state after step t
            if h0 is not None:
                h_all = h_all + np.exp(S[:, None] * a[None, :]) * h0[b, d][None, :]
            yt = np.sum(C[b] * h_all, axis=1)
            if D is not None:
                yt = yt + D[d] * u[b, :, d]
            if z is not None:
                yt = yt * ref_silu(z[b, :, d])
            y[b, :, d] = yt
            h_last[b, d] = h_all[-1] if L > 0 else (0 if h0 is None else h0[b, d])
    return y, h_last


def random_case(rng, batch=2, L=37, Dn=6, N=5, gate=True, with_h0=True, with_D=True,
                with_bias=True):
    """Random small inputs; d_inner != d_state so a transposed index shows."""
    u = rng.standard_normal((batch, L, Dn))
    delta = rng.standard_normal((batch, L, Dn))
    B = rng.standard_normal((batch, L, N))
    C = rng.standard_normal((batch, L, N))
    A = -rng.uniform(0.3, 3.0, size=(Dn, N))
    D = rng.uniform(0.5, 1.5, size=Dn) if with_D else None
    dt = np.exp(rng.uniform(math.log(1e-2), math.log(0.5), size=Dn))
    bias = np.log(np.expm1(dt)) if with_bias else None
    z = rng.standard_normal((batch, L, Dn)) if gate else None
    h0 = rng.standard_normal((batch, Dn, N)) if with_h0 else None
    return dict(u=u, delta=delta, A=A, B=B, C=C, D=D, z=z, bias=bias, h0=h0)


def rel_err(x, r):
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    scale = max(float(np.sqrt(np.mean(r * r))) if r.size else 0.0, 1e-300)
    return float(np.max(np.abs(x - r) / np.maximum(np.abs(r), scale))) if r.size else 0.0


# ----------------------------------------------------------------------------
# pins
# ----------------------------------------------------------------------------

def pin_worked_example(orc):
    """Hand-derived three-step example (tests/golden/worked_example.json)."""
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)
    inp = {k: np.array(v, dtype=np.float64) for k, v in g["inputs"].items()}
    y, h_last = orc.scan(**inp, nthreads=1)
    exp_y = np.array(g["expected"]["y"])
    exp_h = np.array(g["expected"]["h_last"])
    assert np.allclose(y, exp_y, rtol=g["rtol"], atol=0), (y, exp_y)
    assert np.allclose(h_last, exp_h, rtol=g["rtol"], atol=1e-15), (h_last, exp_h)


def pin_brute_force(orc):
    """Recurrence == unrolled O(L^2) sum, with and without gate / h0 / D / bias."""
    rng = np.random.default_rng(11)
    for kw in (dict(), dict(gate=False), dict(with_h0=False), dict(with_D=False),
               dict(with_bias=False), dict(batch=1, L=1, Dn=3, N=4)):
        case = random_case(rng, **kw)
        y, h = orc.scan(**case, nthreads=2)
        yr, hr = brute_force(**case)
        assert rel_err(y, yr) < 1e-11, (kw, rel_err(y, yr))
        assert rel_err(h, hr) < 1e-11, (kw, rel_err(h, hr))


def pin_lti_convolution(orc):
    """Constant Delta, B, C: y = causal conv(K, u) + D u (+ decayed h0), then gate."""
    rng = np.random.default_rng(12)
    batch, L, Dn, N = 2, 96, 4, 6
    A = -rng.uniform(0.05, 2.0, size=(Dn, N))
    dt_const = rng.uniform(0.01, 0.4, size=Dn)
    bias = rng.uniform(-1.0, 1.0, size=Dn)
    # delta chosen so softplus(delta + bias) equals dt_const exactly in real arithmetic
    delta_row = np.log(np.expm1(dt_const)) - bias
    delta = np.broadcast_to(delta_row, (batch, L, Dn)).copy()
    Bc = rng.standard_normal((batch, N))
    Cc = rng.standard_normal((batch, N))
    B = np.broadcast_to(Bc[:, None, :], (batch, L, N)).copy()
    C = np.broadcast_to(Cc[:, None, :], (batch, L, N)).copy()
    u = rng.standard_normal((batch, L, Dn))
    D = rng.uniform(0.5, 1.5, size=Dn)
    z = rng.standard_normal((batch, L, Dn))
    h0 = rng.standard_normal((batch, Dn, N))
    y, h_last = orc.scan(u=u, delta=delta, A=A, B=B, C=C, D=D, z=z, bias=bias, h0=h0)
    k = np.arange(L)
    for b in range(batch):
        for d in range(Dn):
            dl = ref_softplus(delta_row[d] + bias[d])
            abar_pow = np.exp(np.outer(k, dl * A[d]))                    # (L, N): Abar^k
            K = abar_pow @ (Cc[b] * dl * Bc[b])                           # K_k
            conv = np.convolve(u[b, :, d], K)[:L]
            free = np.exp(np.outer(k + 1, dl * A[d])) @ (Cc[b] * h0[b, d])  # C Abar^{t+1} h0
            ref = (conv + free + D[d] * u[b, :, d]) * ref_silu(z[b, :, d])
            assert rel_err(y[b, :, d], ref) < 1e-11, (b, d, rel_err(y[b, :, d], ref))
            h_ref = (np.exp(np.outer(np.arange(L)[::-1], dl * A[d])) * (dl * Bc[b])[None, :]
                     * u[b, :, d][:, None]).sum(0) + np.exp(L * dl * A[d]) * h0[b, d]
            assert rel_err(h_last[b, d], h_ref) < 1e-11


def pin_lti_fft_long(orc):
    """The LTI identity at L = 4096, evaluated with an FFT convolution."""
    rng = np.random.default_rng(13)
    L, Dn, N = 4096, 2, 16
    A = -(np.arange(N) + 1.0)[None, :].repeat(Dn, 0)
    dt_const = np.array([0.003, 0.05])
    delta = np.broadcast_to(np.log(np.expm1(dt_const)), (1, L, Dn)).copy()
    Bc = rng.standard_normal(N)
    Cc = rng.standard_normal(N)
    B = np.broadcast_to(Bc, (1, L, N)).copy()
    C = np.broadcast_to(Cc, (1, L, N)).copy()
    u = rng.standard_normal((1, L, Dn))
    y, _ = orc.scan(u=u, delta=delta, A=A, B=B, C=C)
    nfft = 2 * L
    for d in range(Dn):
        dl = ref_softplus(np.log(np.expm1(dt_const[d])))
        K = np.exp(np.outer(np.arange(L), dl * A[d])) @ (Cc * dl * Bc)
        conv = np.fft.irfft(np.fft.rfft(u[0, :, d], nfft) * np.fft.rfft(K, nfft), nfft)[:L]
        scale = np.sqrt(np.mean(conv ** 2))
        assert np.max(np.abs(y[0, :, d] - conv)) < 1e-9 * max(scale, 1.0)


def pin_zero_input_decay(orc):
    """u = 0: y_t = sum_n C_t[n] exp(A_n S_t) h0[n] * silu(z_t); h_last = exp(A S_L) h0.
    With h0 = 0 as well, y is exactly zero."""
    rng = np.random.default_rng(14)
    case = random_case(rng, L=50)
    case["u"] = np.zeros_like(case["u"])
    y, h_last = orc.scan(**case)
    batch, L, Dn = y.shape
    for b in range(batch):
        for d in range(Dn):
            S = np.cumsum(ref_softplus(case["delta"][b, :, d] + case["bias"][d]))
            decay = np.exp(np.outer(S, case["A"][d]))                     # (L, N)
            ref = (case["C"][b] * decay * case["h0"][b, d]).sum(1) * ref_silu(case["z"][b, :, d])
            assert rel_err(y[b, :, d], ref) < 1e-12
            assert rel_err(h_last[b, d], decay[-1] * case["h0"][b, d]) < 1e-12
            # 0 < Abar <= 1 for A < 0, Delta > 0: each state decays monotonically
            mag = np.abs(decay * case["h0"][b, d])
            assert np.all(np.diff(mag, axis=0) <= 0)
    case["h0"] = None
    y0, h0_last = orc.scan(**case)
    assert np.all(y0 == 0.0) and np.all(h0_last == 0.0)


def pin_special_cases(orc):
    """B = 0 or C = 0 with h0 = 0: y = D u silu(z).  z = 0: y = 0.  Tiny Delta: h_last ~ h0."""
    rng = np.random.default_rng(15)
    case = random_case(rng, with_h0=False)
    expect = case["D"][None, None, :] * case["u"] * ref_silu(case["z"])
    for key in ("B", "C"):
        c = dict(case)
        c[key] = np.zeros_like(case[key])
        y, _ = orc.scan(**c)
        assert rel_err(y, expect) < 1e-13, key
    c = dict(case)
    c["z"] = np.zeros_like(case["z"])
    y, _ = orc.scan(**c)
    assert np.all(y == 0.0)
    # Delta -> 0: softplus(-60) ~ 8.8e-27, the state stays at h0
    c = random_case(rng)
    c["delta"] = np.full_like(c["delta"], -60.0)
    c["bias"] = np.zeros_like(c["bias"])
    _, h_last = orc.scan(**c)
    assert np.allclose(h_last, c["h0"], rtol=1e-20, atol=1e-20)


def pin_split_invariance(orc):
    """scan(0..L) == scan(0..k) then scan(k..L, h0 = h_k), at several k."""
    rng = np.random.default_rng(16)
    case = random_case(rng, L=41)
    y, h = orc.scan(**case)
    for k in (0, 1, 17, 40, 41):
        a = {key: (v[:, :k] if key in ("u", "delta", "B", "C", "z") and v is not None else v)
             for key, v in case.items()}
        ya, ha = orc.scan(**a)
        b = {key: (v[:, k:] if key in ("u", "delta", "B", "C", "z") and v is not None else v)
             for key, v in case.items()}
        b["h0"] = ha
        yb, hb = orc.scan(**b)
        assert np.array_equal(np.concatenate([ya, yb], axis=1), y), k
        assert np.array_equal(hb, h), k


def pin_decode_equals_scan(orc):
    """L chained single-token steps reproduce the scan exactly."""
    rng = np.random.default_rng(17)
    case = random_case(rng, L=23)
    y, h_last = orc.scan(**case)
    h = case["h0"]
    for t in range(case["u"].shape[1]):
        yt, h = orc.step(h, case["u"][:, t], case["delta"][:, t], case["A"], case["B"][:, t],
                         case["C"][:, t], D=case["D"], z=case["z"][:, t], bias=case["bias"])
        assert np.array_equal(yt, y[:, t]), t
    assert np.array_equal(h, h_last)


def pin_linearity_causality(orc):
    """Linear in (u, h0) for fixed delta, B, C, z; y_{<k} ignores inputs at t >= k."""
    rng = np.random.default_rng(18)
    c1 = random_case(rng)
    c2 = dict(c1)
    c2["u"] = rng.standard_normal(c1["u"].shape)
    c2["h0"] = rng.standard_normal(c1["h0"].shape)
    al, be = 0.7, -1.3
    c3 = dict(c1)
    c3["u"] = al * c1["u"] + be * c2["u"]
    c3["h0"] = al * c1["h0"] + be * c2["h0"]
    y1, h1 = orc.scan(**c1)
    y2, h2 = orc.scan(**c2)
    y3, h3 = orc.scan(**c3)
    assert rel_err(y3, al * y1 + be * y2) < 1e-11
    assert rel_err(h3, al * h1 + be * h2) < 1e-11
    k = 20
    c4 = {key: (v.copy() if isinstance(v, np.ndarray) else v) for key, v in c1.items()}
    for key in ("u", "delta", "B", "C", "z"):
        c4[key][:, k:] = rng.standard_normal(c4[key][:, k:].shape)
    y4, _ = orc.scan(**c4)
    assert np.array_equal(y4[:, :k], y1[:, :k])
    assert not np.array_equal(y4[:, k:], y1[:, k:])


def pin_scalar_closed_forms(orc):
    """softplus and silu against closed forms."""
    sp, si = orc.softplus, orc.silu
    assert abs(sp(0.0) - math.log(2.0)) < 1e-16
    assert abs(sp(math.log(math.e - 1.0)) - 1.0) < 1e-15
    for t in (1e-3, 0.1, 5.0):
        assert abs(sp(math.log(math.expm1(t))) - t) < 1e-14 * max(1.0, t)
    assert abs(sp(-50.0) / math.exp(-50.0) - 1.0) < 1e-14
    assert abs(sp(50.0) - 50.0) < 1e-15
    assert abs(sp(-3.0) - math.log1p(math.exp(-3.0))) < 1e-16
    assert abs(sp(7.5) - ref_softplus(7.5)) < 1e-14
    assert si(0.0) == 0.0
    assert abs(si(math.log(3.0)) - 0.75 * math.log(3.0)) < 1e-15
    assert abs(si(-math.log(3.0)) + 0.25 * math.log(3.0)) < 1e-15
    for zz in (-8.0, -0.5, 0.3, 9.0):
        assert abs(si(zz) - ref_silu(zz)) < 1e-14


def pin_empty_and_threads(orc):
    """L = 0 returns h0 as the final state; the thread count does not change bits."""
    rng = np.random.default_rng(19)
    case = random_case(rng, L=0)
    y, h = orc.scan(**case)
    assert y.shape == case["u"].shape and np.array_equal(h, case["h0"])
    case = random_case(rng, L=9, Dn=7)
    y1, h1 = orc.scan(**case, nthreads=1)
    y3, h3 = orc.scan(**case, nthreads=3)
    assert np.array_equal(y1, y3) and np.array_equal(h1, h3)


def _rk4_linear(a, f, h, T, m):
    """Integrate h' = a h + f (constants) over [0, T] with m classical RK4 steps."""
    dt = T / m
    for _ in range(m):
        k1 = a * h + f
        k2 = a * (h + 0.5 * dt * k1) + f
        k3 = a * (h + 0.5 * dt * k2) + f
        k4 = a * (h + dt * k3) + f
        h = h + dt / 6.0 * (k1 + 2 * k2 + 2 * k3 + k4)
    return h


def pin_zoh_samples_the_ode(orc):
    """Zero-order hold is exact for inputs held constant over each step: the ZOH scan's
    states equal a numerical integration (RK4, fine steps) of h' = A h + B_t u_t over
    consecutive intervals of length Delta_t ("State Space Models and Mamba", ZOH;
    "Understanding Mamba" section 12)."""
    rng = np.random.default_rng(31)
    case = random_case(rng, batch=1, L=12, Dn=3, N=4, gate=False, with_D=False)
    y, h_last = orc.scan(**case, zoh=True)
    u, delta, A, B, C, h0, bias = (case[k] for k in ("u", "delta", "A", "B", "C", "h0", "bias"))
    for d in range(3):
        h = h0[0, d].copy()
        for t in range(12):
            dt = ref_softplus(delta[0, t, d] + bias[d])
            h = _rk4_linear(A[d], B[0, t] * u[0, t, d], h, dt, 400)
            assert rel_err(y[0, t, d], np.dot(C[0, t], h)) < 1e-9, (d, t)
        assert rel_err(h_last[0, d], h) < 1e-9, d
    # and it is not the Euler rule
    y_e, _ = orc.scan(**case)
    assert rel_err(y_e, y) > 1e-3


def pin_zoh_limits(orc):
    """A = 0 gives Euler exactly; as Delta -> 0 the two rules agree to first order
    (relative gap ~ |Delta A| / 2 per step)."""
    rng = np.random.default_rng(32)
    case = random_case(rng, L=9, Dn=4, N=3)
    case["A"] = np.zeros_like(case["A"])
    y_z, h_z = orc.scan(**case, zoh=True)
    y_e, h_e = orc.scan(**case)
    assert np.array_equal(y_z, y_e) and np.array_equal(h_z, h_e)
    # tiny steps: one step from a zero state, Bbar_zoh / Bbar_euler = expm1(x)/x, x = Delta A
    case = random_case(rng, batch=1, L=1, Dn=4, N=3, gate=False, with_h0=False, with_D=False)
    case["delta"] = np.full((1, 1, 4), -12.0)   # Delta ~ 6e-6 (with the case's bias)
    case["bias"] = np.zeros(4)
    _, hz = orc.scan(**case, zoh=True)
    _, he = orc.scan(**case)
    dt = ref_softplus(-12.0)
    ratio = hz[0] / he[0]
    expect = 1.0 + dt * case["A"] / 2.0
    assert np.allclose(ratio, expect, rtol=0, atol=1e-9)


def pin_zoh_lti_convolution(orc):
    """Constant Delta, B, C with ZOH: y = causal conv(K, u), K_k = C Abar^k Bbar with
    Bbar = (Abar - 1) / A * B, Abar^k = exp(k Delta A)."""
    rng = np.random.default_rng(33)
    batch, L, Dn, N = 1, 64, 3, 5
    A = -rng.uniform(0.05, 3.0, size=(Dn, N))
    dt_const = rng.uniform(0.05, 0.8, size=Dn)
    delta = np.broadcast_to(np.log(np.expm1(dt_const)), (batch, L, Dn)).copy()
    Bc, Cc = rng.standard_normal(N), rng.standard_normal(N)
    B = np.broadcast_to(Bc, (batch, L, N)).copy()
    C = np.broadcast_to(Cc, (batch, L, N)).copy()
    u = rng.standard_normal((batch, L, Dn))
    y, _ = orc.scan(u=u, delta=delta, A=A, B=B, C=C, zoh=True)
    k = np.arange(L)
    for d in range(Dn):
        dl = ref_softplus(delta[0, 0, d])
        abar = np.exp(dl * A[d])
        K = np.exp(np.outer(k, dl * A[d])) @ (Cc * (abar - 1.0) / A[d] * Bc)
        ref = np.convolve(u[0, :, d], K)[:L]
        assert rel_err(y[0, :, d], ref) < 1e-10, d


def pin_zoh_decode_equals_scan(orc):
    """Chained ZOH decode steps reproduce the ZOH scan exactly."""
    rng = np.random.default_rng(34)
    case = random_case(rng, L=15)
    y, h_last = orc.scan(**case, zoh=True)
    h = case["h0"].copy()
    for t in range(15):
        yt, h = orc.step(h, case["u"][:, t], case["delta"][:, t], case["A"], case["B"][:, t],
                         case["C"][:, t], D=case["D"], z=case["z"][:, t], bias=case["bias"],
                         zoh=True)
        assert np.array_equal(yt, y[:, t]), t
    assert np.array_equal(h, h_last)


PINS = [pin_worked_example, pin_brute_force, pin_lti_convolution, pin_lti_fft_long,
        pin_zero_input_decay, pin_special_cases, pin_split_invariance, pin_decode_equals_scan,
        pin_linearity_causality, pin_scalar_closed_forms, pin_empty_and_threads,
        pin_zoh_samples_the_ode, pin_zoh_limits, pin_zoh_lti_convolution,
        pin_zoh_decode_equals_scan]


# ----------------------------------------------------------------------------
# gradients: pinned by central finite differences of the forward oracle
# ----------------------------------------------------------------------------

def _loss(orc, case, dy, dh_last):
    y, h = orc.scan(**case, nthreads=1)
    return float(np.sum(dy * y) + (np.sum(dh_last * h) if dh_last is not None else 0.0))


def _fd_check(orc, case, dy, dh_last, grads, names, eps=1e-6, tol=2e-7):
    """Every entry of the listed inputs: (L(x + e) - L(x - e)) / 2e against the gradient."""
    key = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
           "z": "dz", "bias": "dbias", "h0": "dh0"}
    for name in names:
        base = case[name]
        g = grads[key[name]]
        worst = 0.0
        scale = max(float(np.max(np.abs(g))), 1e-12)
        for idx in np.ndindex(base.shape):
            h = eps * max(1.0, abs(base[idx]))
            old = base[idx]
            base[idx] = old + h
            lp = _loss(orc, case, dy, dh_last)
            base[idx] = old - h
            lm = _loss(orc, case, dy, dh_last)
            base[idx] = old
            fd = (lp - lm) / (2 * h)
            worst = max(worst, abs(fd - g[idx]) / scale)
        assert worst < tol, (name, worst)


def pin_gradients_finite_differences(orc):
    """Every gradient entry of a small gated problem with h0, D and bias, and of one with
    none of them, against central differences of the forward oracle."""
    rng = np.random.default_rng(41)
    case = random_case(rng, batch=2, L=7, Dn=3, N=4)
    dy = rng.standard_normal(case["u"].shape)
    dh_last = rng.standard_normal(case["h0"].shape)
    g = orc.scan_bwd(dy=dy, dh_last=dh_last, **case)
    _fd_check(orc, case, dy, dh_last, g, ["u", "delta", "A", "B", "C", "D", "z", "bias", "h0"])
    case = random_case(rng, batch=1, L=9, Dn=2, N=3, gate=False, with_h0=False, with_D=False,
                       with_bias=False)
    dy = rng.standard_normal(case["u"].shape)
    g = orc.scan_bwd(dy=dy, **case)
    _fd_check(orc, case, dy, None, g, ["u", "delta", "A", "B", "C"])


def pin_gradient_closed_forms(orc):
    """dD = sum_{b,t} dy g u; with dy = 0 only dh_last flows: dh0 = exp(A S_L) dh_last
    (the adjoint of the exact decay), and du = dy D silu(z) when B = 0."""
    rng = np.random.default_rng(42)
    case = random_case(rng, L=11)
    dy = rng.standard_normal(case["u"].shape)
    g = orc.scan_bwd(dy=dy, **case)
    ref_dD = np.sum(dy * ref_silu(case["z"]) * case["u"], axis=(0, 1))
    assert np.allclose(g["dD"], ref_dD, rtol=1e-12, atol=1e-12)
    dh_last = rng.standard_normal(case["h0"].shape)
    g = orc.scan_bwd(dy=np.zeros_like(dy), dh_last=dh_last, **case)
    for b in range(case["u"].shape[0]):
        for d in range(case["u"].shape[2]):
            S = np.sum(ref_softplus(case["delta"][b, :, d] + case["bias"][d]))
            assert np.allclose(g["dh0"][b, d], np.exp(case["A"][d] * S) * dh_last[b, d],
                               rtol=1e-12, atol=0)
    case["B"] = np.zeros_like(case["B"])
    g = orc.scan_bwd(dy=dy, **case)
    assert np.allclose(g["du"], dy * ref_silu(case["z"]) * case["D"], rtol=1e-12, atol=1e-14)


PINS += [pin_gradients_finite_differences, pin_gradient_closed_forms]


# ----------------------------------------------------------------------------
# Mamba-3 options ("State space models and the Mamba series", jsqmd.com, sections
# 2.1 and 2.2): exponential-trapezoidal input term and data-dependent rotation
# ----------------------------------------------------------------------------

def _shift_in_time(x, first):
    """x_{t-1} along axis 1, with `first` at t = 0."""
    out = np.empty_like(x)
    out[:, 0] = first
    out[:, 1:] = x[:, :-1]
    return out


def pin_trapezoid_lti_kernel(orc):
    """Constant Delta, B, C and lam, no D, gate or h0: y is the causal convolution of u
    with K_0 = lam Delta sum_n C_n B_n and K_k = Delta sum_n C_n B_n (lam Abar_n^k +
    (1 - lam) Abar_n^(k-1)) for k >= 1, plus the look-back input u_prev entering as
    (1 - lam) Delta sum_n C_n B_prev_n Abar_n^t u_prev."""
    rng = np.random.default_rng(51)
    L, Dn, N, lam = 40, 3, 5, 0.37
    u = rng.standard_normal((1, L, Dn))
    dval = rng.standard_normal(Dn)
    delta = np.broadcast_to(dval, (1, L, Dn)).copy()
    Bv, Cv = rng.standard_normal(N), rng.standard_normal(N)
    B = np.broadcast_to(Bv, (1, L, N)).copy()
    C = np.broadcast_to(Cv, (1, L, N)).copy()
    A = -rng.uniform(0.2, 2.0, size=(Dn, N))
    u_prev = rng.standard_normal((1, Dn))
    B_prev = rng.standard_normal((1, N))
    y, _ = orc.scan(u, delta, A, B, C, lam=np.full(u.shape, lam), u_prev=u_prev,
                    B_prev=B_prev)
    k = np.arange(L)
    for d in range(Dn):
        dt = ref_softplus(dval[d])
        ab = np.exp(np.outer(k, dt * A[d]))                     # Abar^k, (L, N)
        ab_m1 = np.vstack([np.zeros(N), ab[:-1]])                # Abar^(k-1), 0 at k = 0
        K = dt * ((lam * ab + (1 - lam) * ab_m1) @ (Cv * Bv))
        ref = np.convolve(u[0, :, d], K)[:L]
        ref = ref + (1 - lam) * dt * (ab @ (Cv * B_prev[0])) * u_prev[0, d]
        assert np.allclose(y[0, :, d], ref, rtol=1e-11, atol=1e-12), d


def pin_trapezoid_limits(orc):
    """lam = 1 is the Euler scan; lam = 0 is the Euler scan of the inputs shifted by one
    step (u_{t-1}, B_{t-1}, starting from u_prev, B_prev) with the same Delta and C."""
    rng = np.random.default_rng(52)
    case = random_case(rng, L=23)
    u_prev = rng.standard_normal((case["u"].shape[0], case["u"].shape[2]))
    B_prev = rng.standard_normal((case["u"].shape[0], case["B"].shape[2]))
    y1, h1 = orc.scan(**case)
    yt, ht = orc.scan(**case, lam=np.ones(case["u"].shape), u_prev=u_prev, B_prev=B_prev)
    assert np.allclose(yt, y1, rtol=1e-14, atol=0) and np.allclose(ht, h1, rtol=1e-14, atol=0)
    c0 = dict(case, D=None)
    y0, h0 = orc.scan(**c0, lam=np.zeros(case["u"].shape), u_prev=u_prev, B_prev=B_prev)
    shifted = dict(c0, u=_shift_in_time(case["u"], u_prev), B=_shift_in_time(case["B"], B_prev))
    ys, hs = orc.scan(**shifted)
    assert np.allclose(h0, hs, rtol=1e-13, atol=1e-14)
    # the readout uses the unshifted gate and C; with D = None y depends on h only
    assert np.allclose(y0, ys, rtol=1e-12, atol=1e-13)


def pin_trapezoid_affine_in_lambda(orc):
    """The state and the output are affine in the mixing coefficients."""
    rng = np.random.default_rng(53)
    case = random_case(rng, L=19)
    shp = case["u"].shape
    l1, l2 = rng.uniform(0, 1, shp), rng.uniform(0, 1, shp)
    a = 0.3
    ya, ha = orc.scan(**case, lam=l1)
    yb, hb = orc.scan(**case, lam=l2)
    ym, hm = orc.scan(**case, lam=a * l1 + (1 - a) * l2)
    assert np.allclose(hm, a * ha + (1 - a) * hb, rtol=1e-12, atol=1e-12)
    assert np.allclose(ym, a * ya + (1 - a) * yb, rtol=1e-11, atol=1e-11)


def pin_trapezoid_split_and_decode(orc):
    """scan(0..L) == scan(0..k) then scan(k..L) continued with (h_k, u_{k-1}, B_{k-1});
    chained decode steps reproduce the scan.  Bitwise."""
    rng = np.random.default_rng(54)
    case = random_case(rng, L=21)
    lam = rng.uniform(0, 1, case["u"].shape)
    up = rng.standard_normal((case["u"].shape[0], case["u"].shape[2]))
    Bp = rng.standard_normal((case["u"].shape[0], case["B"].shape[2]))
    y, h_last = orc.scan(**case, lam=lam, u_prev=up, B_prev=Bp)
    for k in (1, 8, 20):
        first = {key: (v[:, :k] if key in ("u", "delta", "B", "C", "z") else v)
                 for key, v in case.items()}
        rest = {key: (v[:, k:] if key in ("u", "delta", "B", "C", "z") else v)
                for key, v in case.items()}
        y1, h1 = orc.scan(**first, lam=lam[:, :k], u_prev=up, B_prev=Bp)
        rest["h0"] = h1
        y2, h2 = orc.scan(**rest, lam=lam[:, k:], u_prev=case["u"][:, k - 1],
                          B_prev=case["B"][:, k - 1])
        assert np.array_equal(np.concatenate([y1, y2], axis=1), y), k
        assert np.array_equal(h2, h_last), k
    h = case["h0"].copy()
    for t in range(case["u"].shape[1]):
        prev_u = up if t == 0 else case["u"][:, t - 1]
        prev_B = Bp if t == 0 else case["B"][:, t - 1]
        yt, h = orc.step(h, case["u"][:, t], case["delta"][:, t], case["A"], case["B"][:, t],
                         case["C"][:, t], D=case["D"], z=case["z"][:, t], bias=case["bias"],
                         lam=lam[:, t], u_prev=prev_u, B_prev=prev_B)
        assert np.array_equal(yt, y[:, t]), t
    assert np.array_equal(h, h_last)


def _complex_reference(case, theta):
    """The complex state of the pages' continuous form dh/dt = (A + i theta) h +
    (B + i B^) x, with each state pair (2k, 2k+1) read as one complex number
    w_k = h_2k + i h_2k+1 and A equal within a pair: w_t = exp(Delta a) exp(i Delta
    theta_t) w_{t-1} + Delta (B_2k + i B_2k+1) u_t; y_t = sum_k C_2k Re w + C_2k+1 Im w."""
    u, delta, A, B, C = case["u"], case["delta"], case["A"], case["B"], case["C"]
    batch, L, Dn = u.shape
    K = A.shape[1] // 2
    y = np.zeros_like(u)
    h_last = np.zeros((batch, Dn, 2 * K))
    for b in range(batch):
        for d in range(Dn):
            h0 = case["h0"][b, d] if case.get("h0") is not None else np.zeros(2 * K)
            w = h0[0::2] + 1j * h0[1::2]
            a = A[d, 0::2]
            for t in range(L):
                dt = ref_softplus(delta[b, t, d] + case["bias"][d])
                w = np.exp(dt * a) * np.exp(1j * dt * theta[b, t]) * w + \
                    dt * (B[b, t, 0::2] + 1j * B[b, t, 1::2]) * u[b, t, d]
                yt = np.sum(C[b, t, 0::2] * w.real + C[b, t, 1::2] * w.imag) + \
                    case["D"][d] * u[b, t, d]
                y[b, t, d] = yt * ref_silu(case["z"][b, t, d])
            h_last[b, d, 0::2], h_last[b, d, 1::2] = w.real, w.imag
    return y, h_last


def pin_rotation_complex_form(orc):
    """With A equal within each state pair, the rotation is multiplication of the pair,
    read as a complex number, by exp(i Delta theta) (numpy complex arithmetic)."""
    rng = np.random.default_rng(55)
    case = random_case(rng, L=17, N=6)
    case["A"][:, 1::2] = case["A"][:, 0::2]
    theta = rng.uniform(-3, 3, (case["u"].shape[0], 17, 3))
    y, h = orc.scan(**case, theta=theta)
    yr, hr = _complex_reference(case, theta)
    assert np.allclose(y, yr, rtol=1e-11, atol=1e-12)
    assert np.allclose(h, hr, rtol=1e-11, atol=1e-12)


def pin_rotation_pure_and_order(orc):
    """A = 0 and u = 0: each pair turns by the accumulated angle sum_t Delta_t theta_t
    (R(phi) e_1 = (cos phi, sin phi)); distinct decays within a pair, constant Delta and
    theta, u = 0: h_L = (diag(exp(Delta A)) R(Delta theta))^L h0 (numpy matrix power),
    the product in the order the page writes it."""
    rng = np.random.default_rng(56)
    case = random_case(rng, batch=1, L=13, Dn=2, N=4, gate=False, with_D=False)
    case["u"] = np.zeros_like(case["u"])
    theta = rng.uniform(-2, 2, (1, 13, 2))
    zeroA = dict(case, A=np.zeros_like(case["A"]))
    _, h = orc.scan(**zeroA, theta=theta)
    for d in range(2):
        dt = ref_softplus(case["delta"][0, :, d] + case["bias"][d])
        for k in range(2):
            phi = np.sum(dt * theta[0, :, k])
            x, w = case["h0"][0, d, 2 * k], case["h0"][0, d, 2 * k + 1]
            ref = (np.cos(phi) * x - np.sin(phi) * w, np.sin(phi) * x + np.cos(phi) * w)
            assert np.allclose(h[0, d, 2 * k:2 * k + 2], ref, rtol=1e-12, atol=1e-13)
    const = dict(case)
    const["delta"] = np.broadcast_to(case["delta"][:, :1], case["delta"].shape).copy()
    th = np.broadcast_to(theta[:, :1], theta.shape).copy()
    _, h = orc.scan(**const, theta=th)
    for d in range(2):
        dt = ref_softplus(const["delta"][0, 0, d] + case["bias"][d])
        for k in range(2):
            phi = dt * th[0, 0, k]
            R = np.array([[np.cos(phi), -np.sin(phi)], [np.sin(phi), np.cos(phi)]])
            M = np.diag(np.exp(dt * case["A"][d, 2 * k:2 * k + 2])) @ R
            ref = np.linalg.matrix_power(M, 13) @ case["h0"][0, d, 2 * k:2 * k + 2]
            assert np.allclose(h[0, d, 2 * k:2 * k + 2], ref, rtol=1e-11, atol=1e-13)


def pin_rotation_zero_split_decode(orc):
    """theta = 0 is the plain scan; split invariance and decode steps, bitwise."""
    rng = np.random.default_rng(57)
    case = random_case(rng, L=15, N=4)
    y0, h0 = orc.scan(**case)
    yz, hz = orc.scan(**case, theta=np.zeros(case["u"].shape[:2] + (2,)))
    assert np.array_equal(y0, yz) and np.array_equal(h0, hz)
    theta = rng.uniform(-1, 1, case["u"].shape[:2] + (2,))
    y, h_last = orc.scan(**case, theta=theta)
    k = 6
    first = {key: (v[:, :k] if key in ("u", "delta", "B", "C", "z") else v)
             for key, v in case.items()}
    rest = {key: (v[:, k:] if key in ("u", "delta", "B", "C", "z") else v)
            for key, v in case.items()}
    y1, h1 = orc.scan(**first, theta=theta[:, :k])
    rest["h0"] = h1
    y2, h2 = orc.scan(**rest, theta=theta[:, k:])
    assert np.array_equal(np.concatenate([y1, y2], axis=1), y)
    assert np.array_equal(h2, h_last)
    h = case["h0"].copy()
    for t in range(15):
        yt, h = orc.step(h, case["u"][:, t], case["delta"][:, t], case["A"], case["B"][:, t],
                         case["C"][:, t], D=case["D"], z=case["z"][:, t], bias=case["bias"],
                         theta=theta[:, t])
        assert np.array_equal(yt, y[:, t]), t
    assert np.array_equal(h, h_last)


PINS += [pin_trapezoid_lti_kernel, pin_trapezoid_limits, pin_trapezoid_affine_in_lambda,
         pin_trapezoid_split_and_decode, pin_rotation_complex_form, pin_rotation_pure_and_order,
         pin_rotation_zero_split_decode]


# ----------------------------------------------------------------------------
# gradients of the zero-order hold, the trapezoid and the rotation: central finite
# differences of the forward oracle with the same option
# ----------------------------------------------------------------------------

EXT_KEY = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
           "z": "dz", "bias": "dbias", "h0": "dh0", "lam": "dlam", "u_prev": "du_prev",
           "B_prev": "dB_prev", "theta": "dtheta"}


def _ext_loss(orc, case, dy, dh_last):
    y, h = orc.scan(**case, nthreads=1)
    return float(np.sum(dy * y) + np.sum(dh_last * h))


def _ext_fd_check(orc, case, dy, dh_last, g, names, eps=1e-6, tol=3e-7):
    for name in names:
        base = case[name]
        grad = g[EXT_KEY[name]]
        scale = max(float(np.max(np.abs(grad))), 1e-12)
        worst = 0.0
        for idx in np.ndindex(base.shape):
            h = eps * max(1.0, abs(base[idx]))
            old = base[idx]
            base[idx] = old + h
            lp = _ext_loss(orc, case, dy, dh_last)
            base[idx] = old - h
            lm = _ext_loss(orc, case, dy, dh_last)
            base[idx] = old
            worst = max(worst, abs((lp - lm) / (2 * h) - grad[idx]) / scale)
        assert worst < tol, (name, worst)


def _ext_case(rng, *, zoh=False, trap=False, rot=False, prev=True, N=4):
    case = random_case(rng, batch=2, L=6, Dn=3, N=N)
    bl = case["u"].shape[:2]
    if zoh:
        case["zoh"] = True
        case["A"][0, 1] = 0.0          # the A = 0 limit of the zero-order hold
    if trap:
        case["lam"] = rng.uniform(0.0, 1.0, case["u"].shape)
        if prev:
            case["u_prev"] = rng.standard_normal((bl[0], case["u"].shape[2]))
            case["B_prev"] = rng.standard_normal((bl[0], N))
    if rot:
        case["theta"] = rng.uniform(-2.0, 2.0, bl + (N // 2,))
    return case


def pin_option_gradients_finite_differences(orc):
    """Every gradient entry of the zero-order hold, the trapezoid (with and without the
    input before t = 0) and the rotation (alone and with each of the other two) against
    central differences of the forward oracle with that option."""
    rng = np.random.default_rng(71)
    for opts in (dict(zoh=True), dict(trap=True), dict(trap=True, prev=False), dict(rot=True),
                 dict(rot=True, zoh=True), dict(rot=True, trap=True)):
        case = _ext_case(rng, **opts)
        dy = rng.standard_normal(case["u"].shape)
        dh_last = rng.standard_normal(case["h0"].shape)
        g = orc.scan_bwd_ext(dy=dy, dh_last=dh_last, **case)
        names = ["u", "delta", "A", "B", "C", "D", "z", "bias", "h0"]
        names += [k for k in ("lam", "u_prev", "B_prev", "theta") if k in case]
        _ext_fd_check(orc, case, dy, dh_last, g, names)


def pin_option_gradients_reduce_to_euler(orc):
    """Without options the extended gradients are the Euler ones; lam = 1 (no look-back)
    and theta = 0 give them too, with zero gradients for the look-back inputs."""
    rng = np.random.default_rng(72)
    case = random_case(rng, L=9, N=4)
    dy = rng.standard_normal(case["u"].shape)
    dh_last = rng.standard_normal(case["h0"].shape)
    ref = orc.scan_bwd(dy=dy, dh_last=dh_last, **case)
    for extra in ({}, dict(lam=np.ones(case["u"].shape),
                           u_prev=rng.standard_normal((2, 6)),
                           B_prev=rng.standard_normal((2, 4))),
                  dict(theta=np.zeros(case["u"].shape[:2] + (2,)))):
        g = orc.scan_bwd_ext(dy=dy, dh_last=dh_last, **case, **extra)
        for k in ref:
            assert rel_err(g[k], ref[k]) < 1e-12, (sorted(extra), k)
        if "lam" in extra:
            assert np.all(g["du_prev"] == 0.0) and np.all(g["dB_prev"] == 0.0)


PINS += [pin_option_gradients_finite_differences, pin_option_gradients_reduce_to_euler]

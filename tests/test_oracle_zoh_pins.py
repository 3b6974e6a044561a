"""Pins for the oracle's exact zero-order-hold discretisation.

With ZOH, one step is the exact solution of the continuous system
h' = A h + B u over an interval of length delta with B and u held constant
("Illustrated Mamba state space model", "Mathematical basis: structured SSM").
The oracle is checked against a numerical ODE integration of that system
(scipy's DOP853 at tight tolerances), against the continuous steady state
h = -B u / A (which ZOH reproduces exactly whatever the step), against the
delta*B form in the A -> 0 limit, against its own decode step, and its
gradients against central finite differences.
"""
import numpy as np
import pytest
import scipy.integrate

import oracle


def softplus(x):
    return np.logaddexp(0.0, x)


def test_steps_equal_ode_integration():
    rng = np.random.default_rng(1)
    B, D, L, N = 1, 2, 6, 3
    u = rng.standard_normal((B, D, L))
    dt = rng.standard_normal((B, D, L))
    A = -rng.uniform(0.2, 3.0, size=(D, N))
    Bm = rng.standard_normal((B, L, N))
    Cm = rng.standard_normal((B, L, N))
    bias = rng.uniform(-1.0, 0.5, size=D)
    h0 = rng.standard_normal((B, D, N))
    out, hl = oracle.scan(u, dt, A, Bm, Cm, dt_bias=bias, h0=h0, want_h_last=True, zoh=True)
    for d in range(D):
        h = h0[0, d].copy()
        for t in range(L):
            delta = softplus(dt[0, d, t] + bias[d])
            rhs = lambda s, y, t=t: A[d] * y + Bm[0, t] * u[0, d, t]   # held constant over the step
            sol = scipy.integrate.solve_ivp(rhs, (0.0, delta), h, method="DOP853", rtol=1e-12, atol=1e-14)
            h = sol.y[:, -1]
            np.testing.assert_allclose(out[0, d, t], np.dot(Cm[0, t], h), rtol=1e-9, atol=1e-11)
        np.testing.assert_allclose(hl[0, d], h, rtol=1e-9, atol=1e-11)


def test_steady_state_is_exact_for_any_step():
    # constant delta, B and u: h_t -> -B u / A, the fixed point of the continuous system
    D, L, N = 3, 4000, 4
    A = -np.array([[0.5, 1.0, 2.0, 4.0]] * D)
    Bv = np.array([0.3, -1.2, 0.7, 2.0])
    u = np.full((1, D, L), 1.7)
    dt = np.broadcast_to(np.array([-2.0, 0.0, 1.5])[None, :, None], (1, D, L)).copy()  # deltas differ by channel
    Bm = np.broadcast_to(Bv, (1, L, N)).copy()
    _, hl = oracle.scan(u, dt, A, Bm, np.zeros((1, L, N)), want_h_last=True, zoh=True)
    np.testing.assert_allclose(hl[0], np.broadcast_to(-Bv * 1.7 / A[0], (D, N)), rtol=1e-12)
    # the delta*B form has a step-dependent fixed point delta*B*u / (1 - e^{delta A}) instead
    _, he = oracle.scan(u, dt, A, Bm, np.zeros((1, L, N)), want_h_last=True, zoh=False)
    delta = softplus(np.array([-2.0, 0.0, 1.5]))[:, None]
    np.testing.assert_allclose(he[0], delta * Bv * 1.7 / (1 - np.exp(delta * A[0])), rtol=1e-12)


def test_zero_A_limit_equals_delta_B():
    rng = np.random.default_rng(2)
    u, dt = rng.standard_normal((2, 3, 20)), rng.standard_normal((2, 3, 20))
    Bm, Cm = rng.standard_normal((2, 20, 5)), rng.standard_normal((2, 20, 5))
    A = np.zeros((3, 5))
    np.testing.assert_array_equal(oracle.scan(u, dt, A, Bm, Cm, zoh=True), oracle.scan(u, dt, A, Bm, Cm, zoh=False))
    A2 = np.full((3, 5), -1e-9)
    np.testing.assert_allclose(oracle.scan(u, dt, A2, Bm, Cm, zoh=True), oracle.scan(u, dt, A, Bm, Cm), rtol=1e-7,
                               atol=1e-9)


def test_decode_steps_reproduce_zoh_scan():
    rng = np.random.default_rng(3)
    B, D, L, N = 2, 3, 12, 4
    u, dt, z = (rng.standard_normal((B, D, L)) for _ in range(3))
    A = -rng.uniform(0.1, 3.0, (D, N))
    Bm, Cm = rng.standard_normal((B, L, N)), rng.standard_normal((B, L, N))
    bias, Dsk = rng.uniform(-2, 1, D), rng.standard_normal(D)
    ref = oracle.scan(u, dt, A, Bm, Cm, z=z, dt_bias=bias, Dskip=Dsk, zoh=True)
    h = np.zeros((B, D, N))
    for t in range(L):
        o, h = oracle.state_update(h, u[..., t], dt[..., t], A, Bm[:, t], Cm[:, t], z=z[..., t], dt_bias=bias,
                                   Dskip=Dsk, zoh=True)
        np.testing.assert_allclose(o, ref[..., t], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("with_reset", [False, True])
def test_zoh_gradients_finite_differences(with_reset):
    rng = np.random.default_rng(4 + with_reset)
    B, D, L, N = 2, 2, 7, 3
    c = dict(u=rng.standard_normal((B, D, L)), dt_raw=rng.standard_normal((B, D, L)), z=rng.standard_normal((B, D, L)),
             A=-rng.uniform(0.1, 3.0, size=(D, N)), Bm=rng.standard_normal((B, L, N)),
             Cm=rng.standard_normal((B, L, N)), dt_bias=rng.uniform(-3.0, 1.0, size=D), Dskip=rng.standard_normal(D),
             h0=rng.standard_normal((B, D, N)))
    c["A"][0, 0] = -1e-4                      # exercises the small-|delta A| series of d phi / dA
    reset = None
    if with_reset:
        reset = np.zeros((B, L), np.uint8)
        reset[0, 0] = reset[:, 3] = 1
    dout, dhl = rng.standard_normal((B, D, L)), rng.standard_normal((B, D, N))

    def loss():
        out, hl = oracle.scan(c["u"], c["dt_raw"], c["A"], c["Bm"], c["Cm"], z=c["z"], dt_bias=c["dt_bias"],
                              Dskip=c["Dskip"], reset=reset, h0=c["h0"], want_h_last=True, zoh=True)
        return float(np.sum(dout * out) + np.sum(dhl * hl))

    g = oracle.scan_bwd(c["u"], c["dt_raw"], c["A"], c["Bm"], c["Cm"], dout, z=c["z"], dt_bias=c["dt_bias"],
                        Dskip=c["Dskip"], reset=reset, h0=c["h0"], dh_last=dhl, zoh=True)
    names = dict(u="du", dt_raw="d_dt_raw", z="dz", A="dA", Bm="dB", Cm="dC", dt_bias="d_dt_bias", Dskip="dD",
                 h0="dh0")
    for name, gk in names.items():
        x = c[name]
        ref = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            eps = 1e-6 * max(1.0, abs(x[idx]))
            keep = x[idx]
            x[idx] = keep + eps
            fp = loss()
            x[idx] = keep - eps
            fm = loss()
            x[idx] = keep
            ref[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(g[gk], ref, rtol=2e-7, atol=2e-7 * (1 + np.abs(ref).max()), err_msg=name)
